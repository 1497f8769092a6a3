// k_depthwise_rows.hip -- depthwise 3x3 convolution (group = C = M, pads 1,
// stride 1 or 2, no dilation), fp32 or bf16, one row segment per lane.
//
// Y[n, c, oh, ow] = act(b[c] + sum_{kh, kw} W[c, kh, kw] * X[n, c, oh*s - 1 + kh, ow*s - 1 + kw])
// (zero outside the plane): an HBM-bound stencil, no MFMA ("OxiONNX 0.1.7
// Released", Technical Deep Dive item 2, gives depthwise its own kernel).
//
// Work.  A lane owns a segment of V consecutive outputs of a row, for the TR
// output rows of a band of one plane.  The Wo / V lanes that cover a row are
// consecutive lanes of one wave, and a wave holds 64 / (Wo / V) such bands,
// consecutive bands of a plane where the plane has several, so a wave reads
// and writes one contiguous stretch of X and Y.
//
// Memory.  Each lane issues the loads of every input row of its band at
// once (TR + 2 rows for stride 1, 2 TR + 1 for stride 2; one 4-, 8- or
// 16-byte buffer load per row: its segment's V * s input columns), so a
// wave keeps TR + 2 or more KB in flight with no LDS and no barrier.  A row
// above or below the plane, and every load of a lane without a band, reads
// at an offset past the tensor, which the buffer load returns as zeros.
// The rows that two bands share are read by both; the second read is an L2
// hit.
//
// Halo.  The column left of a segment is the last input of the left
// neighbour lane's segment, the column right of it the first input of the
// right neighbour's; both move between lanes with whole-wave DPP shifts (one
// v_mov_dpp each) and are zero at the plane's edges (the first and last lane
// of a band row).
//
// Arithmetic, fp32: 9 FMAs per output.  bf16 rows of odd width: one output
// per lane (2-byte loads), widened to fp32 and 9 FMAs per output.  Other
// bf16: the inputs stay packed as
// pairs at even columns, and v_dot2_f32_bf16 (two bf16 products and an fp32
// addend) takes two taps per instruction: an output at an even column is
// (w1, w2).(x[c], x[c+1]) + (0, w0).(x[c-2], x[c-1]); one at an odd column is
// (w0, w1).(x[c-1], x[c]) + (w2, 0).(x[c+1], x[c+2]) -- 6 instructions per
// output, no widening.  Bias is the first addend; the activation and the
// bf16 rounding (v_cvt_pk_bf16_f32, nearest even) close each row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "engine.hpp"

namespace ox {

namespace dwr {

constexpr uint32_t kOutside = 0x80000000u;   // a load offset past any X this kernel takes (< 2^31 bytes)

struct Plan {
  int V, TR;         // outputs per lane per row, output rows per band
  int nseg;          // lanes per band row: Wo / V
  int gpw;           // bands per wave: 64 / nseg
  int nb;            // bands per plane
  int bands;         // N * C * nb
  int grid;          // blocks of 4 waves
  uint32_t x_bytes;  // bytes of X
  FastDiv nseg_div, nb_div, c_div;
};

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// acc + (a.lo * b.lo + a.hi * b.hi), products of bf16 pairs, fp32 sum
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, a), __builtin_bit_cast(bf16x2v_t, b), acc,
                                         false);
}

// v from lane l - 1 (lane 0: zero) / from lane l + 1 (lane 63: zero)
__device__ __forceinline__ uint32_t from_left(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xf, 0xf, false);   // wave_shr:1
}
__device__ __forceinline__ uint32_t from_right(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, false);   // wave_shl:1
}

// ND dwords of a segment (ND = 0: one 2-byte element, zero-extended)
template <int ND>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* d) {
  if constexpr (ND == 0) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (ND == 1) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (ND == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    d[0] = v[0];
    d[1] = v[1];
  } else {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    d[0] = v[0];
    d[1] = v[1];
    d[2] = v[2];
    d[3] = v[3];
  }
}

template <int DT, int ST, int V, int TR>
__global__ __launch_bounds__(kThreads) void dw3x3_rows(const ConvArgs a, const Plan pl) {
  constexpr int E = DT == DT_F32 ? 4 : 2;
  constexpr int LB = V * ST * E;                         // bytes of a lane's input row segment
  constexpr int ND = LB / 4;                             // its dwords (0: one bf16 element)
  constexpr int NR = ND > 0 ? ND : 1;                    // registers of a row segment
  constexpr int RIN = ST == 1 ? TR + 2 : 2 * TR + 1;     // input rows of a band
  // bf16, stride 1, one output per lane: rows of odd width (pairs would
  // straddle rows), arithmetic in fp32 on the widened elements
  constexpr bool WIDE1 = DT == DT_BF16 && ST == 1 && V == 1;
  static_assert(LB == 4 || LB == 8 || LB == 16 || (WIDE1 && LB == 2), "segment load width");
  static_assert(DT == DT_F32 || ST == 2 || V % 2 == 0 || WIDE1, "bf16 stride-1 segments hold whole pairs");
  typedef typename std::conditional<DT == DT_F32, float, uint16_t>::type T;

  const int lane = threadIdx.x & 63;
  const int wv = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int g = (int)fdiv(pl.nseg_div, (uint32_t)lane);  // the lane's band in the wave
  const int j = lane - g * pl.nseg;                      // its segment in the row
  const int gi = wv * pl.gpw + g;
  const bool valid = g < pl.gpw && gi < pl.bands;
  const int gc = valid ? gi : 0;
  const int p = (int)fdiv(pl.nb_div, (uint32_t)gc);      // plane
  const int oh0 = (gc - p * pl.nb) * TR;                 // first output row of the band
  const int c = p - (int)fdiv(pl.c_div, (uint32_t)p) * a.C;
  const int H = a.H, Ho = a.Ho, Wo = a.Wo;

  // every input row of the band
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.X), (short)0, (int)pl.x_bytes, 0x00020000);
  const uint32_t seg0 = (uint32_t)p * (uint32_t)(H * a.W * E) + (uint32_t)(j * LB);
  const uint32_t rowb = (uint32_t)(a.W * E);
  const int r0 = oh0 * ST - 1;
  uint32_t d[RIN][NR];
#pragma unroll
  for (int rr = 0; rr < RIN; ++rr) {
    const int r = r0 + rr;
    const bool in = valid && r >= 0 && r < H;
    load_row<ND>(xr, in ? seg0 + (uint32_t)r * rowb : kOutside, d[rr]);
  }

  // taps and bias of channel c, issued behind the rows so that both arrive
  // in one round trip (the bias through a raw buffer of 0 bytes when there
  // is none: no branch, whose merge would make the rows wait for it)
  float wf[9], bias;
  uint32_t wb[9];
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.bias), (short)0, a.bias ? a.C * E : 0, 0x00020000);
  if constexpr (DT == DT_F32) {
    const float* w = (const float*)a.Wt + c * 9;
#pragma unroll
    for (int t = 0; t < 9; ++t) wf[t] = w[t];
    bias = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(br, (uint32_t)c * 4u, 0, 0));
  } else {
    const uint16_t* w = (const uint16_t*)a.Wt + c * 9;
#pragma unroll
    for (int t = 0; t < 9; ++t) wb[t] = w[t];
    bias = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(br, (uint32_t)c * 2u, 0, 0));
  }

  // halo columns of each input row (zero at the plane's left / right edge)
  const bool first = j == 0, last = j == pl.nseg - 1;
  uint32_t hl[RIN], hr[RIN];
#pragma unroll
  for (int rr = 0; rr < RIN; ++rr) {
    const uint32_t l = from_left(d[rr][NR - 1]);
    hl[rr] = first ? 0u : l;
    if constexpr (ST == 1) {
      const uint32_t r = from_right(d[rr][0]);
      hr[rr] = last ? 0u : r;
    }
  }

  // bf16 tap pairs per kernel row: (w1, w2), (0, w0), (w0, w1), (w2, 0)
  // (one output per lane: the taps widened instead)
  uint32_t pa[3], pb[3], pc[3], pd[3];
  if constexpr (WIDE1) {
#pragma unroll
    for (int t = 0; t < 9; ++t) wf[t] = bf16_to_f32((uint16_t)wb[t]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
      pa[kh] = wb[3 * kh + 1] | (wb[3 * kh + 2] << 16);
      pb[kh] = wb[3 * kh] << 16;
      pc[kh] = wb[3 * kh] | (wb[3 * kh + 1] << 16);
      pd[kh] = wb[3 * kh + 2];
    }
  }

  T* Y = (T*)a.Y;
  const bool vec_ok = (((uintptr_t)a.Y) & (V * E - 1)) == 0;
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int o = 0; o < TR; ++o) {
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = bias;
#pragma unroll
      for (int kh = 0; kh < 3; ++kh) {
        const int rr = ST * o + kh;
        const uint32_t* x = d[rr];
        if constexpr (WIDE1) {
          acc[0] = fmaf(wf[3 * kh], __uint_as_float(hl[rr] << 16), acc[0]);
          acc[0] = fmaf(wf[3 * kh + 1], __uint_as_float(x[0] << 16), acc[0]);
          acc[0] = fmaf(wf[3 * kh + 2], __uint_as_float(hr[rr] << 16), acc[0]);
        } else if constexpr (DT == DT_BF16 && ST == 1) {
#pragma unroll
          for (int m = 0; m < ND; ++m) {
            acc[2 * m] = dot2(x[m], pa[kh], acc[2 * m]);
            acc[2 * m] = dot2(m > 0 ? x[m - 1] : hl[rr], pb[kh], acc[2 * m]);
            acc[2 * m + 1] = dot2(x[m], pc[kh], acc[2 * m + 1]);
            acc[2 * m + 1] = dot2(m < ND - 1 ? x[m + 1] : hr[rr], pd[kh], acc[2 * m + 1]);
          }
        } else if constexpr (DT == DT_BF16) {
          // stride 2: output i covers columns 2i - 1 .. 2i + 1; pair i is (2i, 2i + 1)
#pragma unroll
          for (int i = 0; i < V; ++i) {
            acc[i] = dot2(x[i], pa[kh], acc[i]);
            acc[i] = dot2(i > 0 ? x[i - 1] : hl[rr], pb[kh], acc[i]);
          }
        } else if constexpr (ST == 1) {
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const float xl = __uint_as_float(i > 0 ? x[i - 1] : hl[rr]);
            const float xr_ = __uint_as_float(i < V - 1 ? x[i + 1] : hr[rr]);
            acc[i] = fmaf(wf[3 * kh], xl, acc[i]);
            acc[i] = fmaf(wf[3 * kh + 1], __uint_as_float(x[i]), acc[i]);
            acc[i] = fmaf(wf[3 * kh + 2], xr_, acc[i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const float xl = __uint_as_float(i > 0 ? x[2 * i - 1] : hl[rr]);
            acc[i] = fmaf(wf[3 * kh], xl, acc[i]);
            acc[i] = fmaf(wf[3 * kh + 1], __uint_as_float(x[2 * i]), acc[i]);
            acc[i] = fmaf(wf[3 * kh + 2], __uint_as_float(x[2 * i + 1]), acc[i]);
          }
        }
      }
      const int oh = oh0 + o;
      if (valid && oh < Ho) {
        T* dst = Y + ((size_t)p * Ho + oh) * Wo + j * V;
        if constexpr (DT == DT_F32) {
          float v[V];
#pragma unroll
          for (int i = 0; i < V; ++i) v[i] = act_c<ACT>(acc[i]);
          if (vec_ok) {
            if constexpr (V == 4) *(f32x4_t*)dst = f32x4_t{v[0], v[1], v[2], v[3]};
            else if constexpr (V == 2) *(f32x2_t*)dst = f32x2_t{v[0], v[1]};
            else dst[0] = v[0];
          } else {
#pragma unroll
            for (int i = 0; i < V; ++i) dst[i] = v[i];
          }
        } else {
          if constexpr (V == 1) {
            dst[0] = (uint16_t)(pack_bf16x2(act_c<ACT>(acc[0]), 0.f) & 0xffffu);
          } else {
            uint32_t q[V / 2];
#pragma unroll
            for (int i = 0; i < V / 2; ++i) q[i] = pack_bf16x2(act_c<ACT>(acc[2 * i]), act_c<ACT>(acc[2 * i + 1]));
            if (vec_ok) {
              if constexpr (V == 8) *(u32x4_t*)dst = u32x4_t{q[0], q[1], q[2], q[3]};
              else if constexpr (V == 4) *(u32x2_t*)dst = u32x2_t{q[0], q[1]};
              else *(uint32_t*)dst = q[0];
            } else {
#pragma unroll
              for (int i = 0; i < V / 2; ++i) {
                dst[2 * i] = (uint16_t)(q[i] & 0xffffu);
                dst[2 * i + 1] = (uint16_t)(q[i] >> 16);
              }
            }
          }
        }
      }
    }
  });
}

// The plan for a geometry, or false where this kernel does not apply.
bool make_plan(const ConvArgs& a, Plan* out) {
  if (a.dt != DT_F32 && a.dt != DT_BF16) return false;
  if (!(a.group == a.C && a.M == a.C && a.kH == 3 && a.kW == 3 && a.pt == 1 && a.pl == 1 && a.dh == 1 &&
        a.dw == 1 && a.sh == a.sw && (a.sh == 1 || a.sh == 2) && a.Ho == (a.H + 2 - 3) / a.sh + 1 &&
        a.Wo == (a.W + 2 - 3) / a.sw + 1))
    return false;
  if (a.N <= 0 || a.C <= 0 || a.Ho <= 0 || a.Wo <= 0) return false;
  const int s = a.sh, E = a.dt == DT_F32 ? 4 : 2;
  const bool bf = a.dt == DT_BF16;
  // a segment's input columns are V * s consecutive columns of one row: the
  // row holds Wo * s of them (stride 2 needs an even width; bf16 stride 1
  // keeps pairs at even columns, so an even width too)
  if (a.W != a.Wo * s) return false;
  // bf16 at stride 1: pairs on even widths, one output per lane on odd ones
  const bool odd1 = bf && s == 1 && a.W % 2 != 0;
  const int64_t P = (int64_t)a.N * a.C, HW = (int64_t)a.H * a.W;
  if (P * HW * E >= ((int64_t)1 << 31) || P * a.Ho * a.Wo >= ((int64_t)1 << 31)) return false;
  int vmax = 8;
  if (const char* e = getenv("OX_DWR_V")) vmax = atoi(e);
  Plan p;
  p.V = 0;
  for (int V = odd1 ? 1 : 8; V >= 1; V /= 2) {
    const int lb = V * s * E;
    if (V > vmax || lb > 16 || (lb < 4 && !odd1) || (bf && s == 1 && V % 2 && !odd1)) continue;
    if (a.Wo % V || a.Wo / V > 64 || ((uintptr_t)a.X % lb)) continue;
    p.V = V;
    break;
  }
  if (!p.V) return false;
  p.nseg = a.Wo / p.V;
  p.gpw = 64 / p.nseg;
  // four output rows per band: with inputs coming from HBM, four beat eight
  // on every MobileNetV2 layer of 14 rows or more (more, shorter-lived
  // waves; the extra halo rows are L2 hits); eight where they cover a plane
  // of 5 to 8 rows in one band (the 7x7 layers: 11.5 -> 10.3 us bf16); eight
  // on request
  p.TR = a.Ho > 4 && a.Ho <= 8 ? 8 : 4;
  if (const char* e = getenv("OX_DWR_TR")) p.TR = atoi(e) == 8 ? 8 : 4;
  p.nb = (a.Ho + p.TR - 1) / p.TR;
  if (P * p.nb >= ((int64_t)1 << 31)) return false;
  p.bands = (int)(P * p.nb);
  const int64_t nw = (P * p.nb + p.gpw - 1) / p.gpw;
  p.grid = (int)((nw + kThreads / 64 - 1) / (kThreads / 64));
  p.x_bytes = (uint32_t)(P * HW * E);
  p.nseg_div = make_fastdiv((uint32_t)p.nseg);
  p.nb_div = make_fastdiv((uint32_t)p.nb);
  p.c_div = make_fastdiv((uint32_t)a.C);
  *out = p;
  return true;
}

template <int DT, int ST, int V>
int launch_v(const ConvArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid(p.grid);
  if (p.TR == 8) hipLaunchKernelGGL((dw3x3_rows<DT, ST, V, 8>), grid, dim3(kThreads), 0, s, a, p);
  else hipLaunchKernelGGL((dw3x3_rows<DT, ST, V, 4>), grid, dim3(kThreads), 0, s, a, p);
  return (int)hipGetLastError();
}

int launch(const ConvArgs& a, const Plan& p, hipStream_t s) {
  if (a.dt == DT_BF16) {
    if (a.sh == 1) {
      if (p.V == 8) return launch_v<DT_BF16, 1, 8>(a, p, s);
      if (p.V == 4) return launch_v<DT_BF16, 1, 4>(a, p, s);
      if (p.V == 2) return launch_v<DT_BF16, 1, 2>(a, p, s);
      return launch_v<DT_BF16, 1, 1>(a, p, s);
    }
    if (p.V == 4) return launch_v<DT_BF16, 2, 4>(a, p, s);
    if (p.V == 2) return launch_v<DT_BF16, 2, 2>(a, p, s);
    return launch_v<DT_BF16, 2, 1>(a, p, s);
  }
  if (a.sh == 1) {
    if (p.V == 4) return launch_v<DT_F32, 1, 4>(a, p, s);
    if (p.V == 2) return launch_v<DT_F32, 1, 2>(a, p, s);
    return launch_v<DT_F32, 1, 1>(a, p, s);
  }
  if (p.V == 2) return launch_v<DT_F32, 2, 2>(a, p, s);
  return launch_v<DT_F32, 2, 1>(a, p, s);
}

}  // namespace dwr

bool depthwise_rows_applicable(const ConvArgs& a) {
  dwr::Plan p;
  return dwr::make_plan(a, &p);
}

int launch_conv_depthwise_rows(const ConvArgs& a, void* stream) {
  dwr::Plan p;
  if (!dwr::make_plan(a, &p)) return (int)hipErrorInvalidValue;
  return dwr::launch(a, p, (hipStream_t)stream);
}

const char* conv_depthwise_rows_describe(const ConvArgs& a, char* buf, int cap) {
  dwr::Plan p;
  if (!dwr::make_plan(a, &p)) return "";
  snprintf(buf, cap, "V=%d TR=%d seg=%d bands/wave=%d bands/plane=%d grid=%d", p.V, p.TR, p.nseg, p.gpw, p.nb,
           p.grid);
  return buf;
}

}  // namespace ox
