// k_conv_patch.hip -- implicit-GEMM 3x3 convolution, bf16, with the input
// patch staged once per channel chunk.
//
// The generic implicit GEMM gathers every (channel, tap) element of its
// operand from global memory, i.e. each input value is fetched once per tap.
// Here a block owns BM output channels and a band of TR output rows (or IMB
// whole images) and, for each chunk of 32 input channels:
//   * stages the input band (with its halo, zero-filled once) in LDS in a
//     channel-contiguous layout: one 80-byte cell per input position holds the
//     32 channels (64 bytes) plus 16 bytes of bank padding.  NCHW rows are
//     read with the widest aligned vector loads the plane size allows and
//     transposed in registers, eight channels at a time;
//   * stages the weights of the chunk tap-major: W[m, c, kh, kw] is read as
//     it lies in memory (8 channels x 9 taps = 9 aligned 16-byte loads) and
//     permuted in registers so that each tap holds its 32 channels
//     contiguously;
//   * runs 9 taps x (BM/16) x (tiles of 16 pixels) MFMA 16x16x32 bf16: for tap
//     (kh, kw) the operand of output pixel p is simply the cell at p's patch
//     position plus a tap offset, so both MFMA fragments are single 128-bit
//     LDS reads.
// Columns of the patch are stored de-interleaved by stride phase (all
// positions with pc % s == 0 first), so consecutive output pixels read
// consecutive cells for stride 2 as well as stride 1.
// The next chunk's global loads are issued before the current chunk's MFMAs
// and land in registers; one LDS buffer, two barriers per chunk.
#include <algorithm>

#include "engine.hpp"

namespace ox {

struct PatchPlan {
  int TR;       // output rows per block (per image)
  int IMB;      // images per block (> 1 only when TR == Ho)
  int PR;       // patch rows per image
  int PWs;      // patch columns per stride phase
  int PWt;      // patch row length in cells (s_w * PWs)
  int NT;       // 16-pixel tiles per block
  int nrb;      // row blocks per image
  int nib;      // image blocks
  int npos;     // cells in the patch (IMB * PR * PWt)
  int PW;       // patch columns actually used
  int VW;       // elements per global vector load of an input row span
  int units;    // patch staging units (8 channels x VW positions) per image, per octet
};

namespace {

constexpr int kCell = 80;     // bytes per patch cell
// patch staging units per thread (upper bound): one 8-channel x 8-position
// unit already takes 32 registers, narrower vectors allow two
constexpr int upt(int VW) { return VW == 8 ? 1 : 2; }

template <int VW> struct VecT;
template <> struct VecT<8> { typedef u32x4_t T; };
template <> struct VecT<4> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct VecT<2> { typedef uint32_t T; };
template <> struct VecT<1> { typedef uint16_t T; };

template <int VW>
__device__ __forceinline__ uint16_t lane_elem(const typename VecT<VW>::T& v, int e) {
  if constexpr (VW == 8) {
    const uint32_t w = v[e >> 1];
    return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
  } else if constexpr (VW == 4) {
    const uint32_t w = v[e >> 1];
    return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
  } else if constexpr (VW == 2) {
    return (uint16_t)((e & 1) ? (v >> 16) : (v & 0xffffu));
  } else {
    return v;
  }
}

template <int BM, int FN, int VW>
__global__ __launch_bounds__(kThreads, 2) void conv3x3_patch_bf16(const ConvArgs a, const PatchPlan pp) {
  constexpr int KK = 9;
  constexpr int FM = BM / 16;
  constexpr int AROW = KK * 64 + 16;
  constexpr int WUNITS = BM * 4 / kThreads;      // weight staging units per thread
  typedef typename VecT<VW>::T VT;
  constexpr int kUPT = upt(VW);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* As = smem;
  char* Ps = smem + BM * AROW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int bx = blockIdx.x;
  const int img0 = (bx / pp.nrb) * pp.IMB;
  const int oh0 = (bx - (bx / pp.nrb) * pp.nrb) * pp.TR;
  const int rows_here = min(pp.TR, a.Ho - oh0);
  const int imgs_here = min(pp.IMB, a.N - img0);
  const int H = a.H, W = a.W, HW = H * W;
  const int C = a.C, M = a.M;
  const int K = C * KK;
  const int ih_base = oh0 * a.sh - a.pt;
  const int ihs = max(0, ih_base), ihe = min(H, ih_base + pp.PR);
  const int fs = (ihs * W / VW) * VW;
  const int nvec = ihe > ihs ? ((ihe * W + VW - 1) / VW * VW - fs) / VW : 0;
  const int units = imgs_here * 4 * nvec;
  const uint16_t* X = (const uint16_t*)a.X;
  const uint16_t* Wt = (const uint16_t*)a.Wt;

  // zero the whole patch once: halo cells are never written again
  for (int i = tid; i < pp.npos * (kCell / 16); i += kThreads)
    *(u32x4_t*)(Ps + i * 16) = u32x4_t{0u, 0u, 0u, 0u};

  // this lane's output pixels (one per N-tile the wave owns)
  int pbase[FN];
  bool pvalid[FN];
  int pimg[FN], prow[FN], pcol[FN];
  const int ppi = pp.TR * a.Wo;   // pixel slots per image
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int q = (wave + 4 * f) * 16 + lr;
    const int i = q / ppi;
    const int rem = q - i * ppi;
    const int r = rem / a.Wo;
    const int c = rem - r * a.Wo;
    pvalid[f] = (wave + 4 * f < pp.NT) && i < imgs_here && r < rows_here;
    pimg[f] = i;
    prow[f] = r;
    pcol[f] = c;
    pbase[f] = pvalid[f] ? (i * pp.PR + r * a.sh) * pp.PWt + c : 0;
  }
  // tap offsets in cells
  int toff[KK];
#pragma unroll
  for (int t = 0; t < KK; ++t) {
    const int kh = t / 3, kw = t % 3;
    const int cw = kw * a.dw;
    toff[t] = kh * a.dh * pp.PWt + (cw % a.sw) * pp.PWs + cw / a.sw;
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wreg[WUNITS][KK];
  VT xreg[kUPT][8];

  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int k = 0; k < WUNITS; ++k) {
      const int u = tid + k * kThreads;
      const int m = u >> 2, oct = u & 3;
      if (m0 + m < M) {
        const uint16_t* src = Wt + (int64_t)(m0 + m) * K + (c0 + oct * 8) * KK;
#pragma unroll
        for (int j = 0; j < KK; ++j) wreg[k][j] = *(const u32x4_t*)(src + 8 * j);
      } else {
#pragma unroll
        for (int j = 0; j < KK; ++j) wreg[k][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < kUPT; ++k) {
      const int u = tid + k * kThreads;
      if (u < units) {
        const int i = u / (4 * nvec);
        const int rem = u - i * 4 * nvec;
        const int oct = rem / nvec;
        const int v = rem - oct * nvec;
        const uint16_t* src = X + ((int64_t)(img0 + i) * C + c0 + oct * 8) * HW + fs + v * VW;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) xreg[k][ch] = *(const VT*)(src + (int64_t)ch * HW);
      }
    }
  };

  auto store_chunk = [&]() {
#pragma unroll
    for (int k = 0; k < WUNITS; ++k) {
      const int u = tid + k * kThreads;
      const int m = u >> 2, oct = u & 3;
      char* dst = As + m * AROW + oct * 16;
#pragma unroll
      for (int t = 0; t < KK; ++t) {
        // tap t of channels oct*8 .. oct*8+7: elements c*9 + t of the 72 loaded
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e0 = (2 * j) * KK + t, e1 = (2 * j + 1) * KK + t;
          const uint32_t w0 = wreg[k][e0 >> 3][(e0 & 7) >> 1];
          const uint32_t w1 = wreg[k][e1 >> 3][(e1 & 7) >> 1];
          const uint32_t lo = (e0 & 1) ? (w0 >> 16) : (w0 & 0xffffu);
          const uint32_t hi = (e1 & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
          d[j] = lo | hi;
        }
        *(u32x4_t*)(dst + t * 64) = u32x4_t{d[0], d[1], d[2], d[3]};
      }
    }
#pragma unroll
    for (int k = 0; k < kUPT; ++k) {
      const int u = tid + k * kThreads;
      if (u < units) {
        const int i = u / (4 * nvec);
        const int rem = u - i * 4 * nvec;
        const int oct = rem / nvec;
        const int v = rem - oct * nvec;
        const int f0 = fs + v * VW;
        int ih = f0 / W;
        int iw = f0 - ih * W;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          const int pc = iw + a.pl;
          if (ih >= ihs && ih < ihe && pc < pp.PW) {
            const int pr = ih - ih_base;
            const int cell = (i * pp.PR + pr) * pp.PWt + (pc % a.sw) * pp.PWs + pc / a.sw;
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              d[j] = (uint32_t)lane_elem<VW>(xreg[k][2 * j], e) |
                     ((uint32_t)lane_elem<VW>(xreg[k][2 * j + 1], e) << 16);
            *(u32x4_t*)(Ps + cell * kCell + oct * 16) = u32x4_t{d[0], d[1], d[2], d[3]};
          }
          if (++iw == W) {
            iw = 0;
            ++ih;
          }
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
#pragma unroll
    for (int t = 0; t < KK; ++t) {
      u32x4_t af[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *(const u32x4_t*)(As + (fm * 16 + lr) * AROW + t * 64 + lg * 16);
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        if (wave + 4 * f < pp.NT) {
          const u32x4_t bfr = *(const u32x4_t*)(Ps + (pbase[f] + toff[t]) * kCell + lg * 16);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) Mma<DT_BF16>::run(acc[fm][f], af[fm], bfr);
        }
      }
    }
  }

  // epilogue: bias, activation, round to bf16
  const uint16_t* bias = (const uint16_t*)a.bias;
  uint16_t* Y = (uint16_t*)a.Y;
  const int HoWo = a.Ho * a.Wo;
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    if (!pvalid[f]) continue;
    const int64_t pix = (int64_t)(oh0 + prow[f]) * a.Wo + pcol[f];
    const int64_t img = img0 + pimg[f];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + fm * 16 + lg * 4 + i;
        if (m < M) {
          float v = acc[fm][f][i];
          if (bias) v += bf16_to_f32(bias[m]);
          Y[(img * M + m) * HoWo + pix] = f32_to_bf16(apply_act(a.act, v));
        }
      }
  }
}

constexpr int kLdsMax = 160 * 1024;

int lds_bytes(int BM, const PatchPlan& p) { return BM * (9 * 64 + 16) + p.npos * kCell; }

// Fill the geometry of a plan with TR output rows and IMB images per block.
PatchPlan make(const ConvArgs& a, int TR, int IMB) {
  PatchPlan p;
  p.TR = TR;
  p.IMB = IMB;
  p.PR = (TR - 1) * a.sh + 2 * a.dh + 1;
  p.PW = (a.Wo - 1) * a.sw + 2 * a.dw + 1;
  p.PWs = (p.PW + a.sw - 1) / a.sw;
  p.PWt = p.PWs * a.sw;
  p.NT = (IMB * TR * a.Wo + 15) / 16;
  p.nrb = (a.Ho + TR - 1) / TR;
  p.nib = (a.N + IMB - 1) / IMB;
  p.npos = IMB * p.PR * p.PWt;
  const int HW = a.H * a.W;
  p.VW = (HW % 8 == 0) ? 8 : (HW % 4 == 0) ? 4 : (HW % 2 == 0) ? 2 : 1;
  // staging units for a full block: images x 4 octets x vectors of the row span
  const int span = std::min(a.H, p.PR) * a.W;
  p.units = IMB * 4 * ((span + 2 * p.VW - 2) / p.VW);
  return p;
}

bool plan_ok(const ConvArgs& a, int BM, const PatchPlan& p) {
  return p.NT <= 16 && lds_bytes(BM, p) <= kLdsMax && p.units <= upt(p.VW) * kThreads &&
         p.nrb * p.nib < (1 << 30) && ((int64_t)p.IMB * a.N >= 1);
}

// Pick rows/images per block: about 112-224 pixels per block, as many blocks
// as possible for 256 CUs, within the LDS and staging limits.
bool choose(const ConvArgs& a, int* BMo, PatchPlan* out) {
  const int BM = 64;
  PatchPlan best;
  bool found = false;
  double best_score = -1;
  for (int IMB = 1; IMB <= 4; ++IMB) {
    for (int TR = 1; TR <= a.Ho; ++TR) {
      if (IMB > 1 && TR != a.Ho) continue;
      PatchPlan p = make(a, TR, IMB);
      if (!plan_ok(a, BM, p)) continue;
      const double slots = p.NT * 16.0;
      const double used = (double)IMB * TR * a.Wo;
      const double eff = used / slots;                       // tile fill
      const double blocks = (double)p.nrb * p.nib * ((a.M + BM - 1) / BM);
      const double fill = std::min(1.0, blocks / 512.0);     // two blocks per CU
      const double reuse = std::min(1.0, p.NT / 14.0);       // LDS reads per MFMA
      const double score = eff * fill * (0.6 + 0.4 * reuse);
      if (score > best_score + 1e-9) {
        best_score = score;
        best = p;
        found = true;
      }
    }
  }
  *BMo = BM;
  *out = best;
  return found;
}

template <int BM, int FN>
int launch_vw(const ConvArgs& a, const PatchPlan& p, hipStream_t s) {
  dim3 grid(p.nrb * p.nib, (a.M + BM - 1) / BM, 1);
  const int bytes = lds_bytes(BM, p);
  switch (p.VW) {
    case 8: hipLaunchKernelGGL((conv3x3_patch_bf16<BM, FN, 8>), grid, dim3(kThreads), bytes, s, a, p); break;
    case 4: hipLaunchKernelGGL((conv3x3_patch_bf16<BM, FN, 4>), grid, dim3(kThreads), bytes, s, a, p); break;
    case 2: hipLaunchKernelGGL((conv3x3_patch_bf16<BM, FN, 2>), grid, dim3(kThreads), bytes, s, a, p); break;
    default: hipLaunchKernelGGL((conv3x3_patch_bf16<BM, FN, 1>), grid, dim3(kThreads), bytes, s, a, p); break;
  }
  return (int)hipGetLastError();
}

}  // namespace

bool conv_patch_applicable(const ConvArgs& a) {
  if (a.dt != DT_BF16 || a.group != 1 || a.kH != 3 || a.kW != 3 || a.C % 32 != 0) return false;
  if (!a.w_vec || (((uintptr_t)a.X) & 15) != 0) return false;
  int BM;
  PatchPlan p;
  return choose(a, &BM, &p);
}

int launch_conv_patch(const ConvArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  int BM;
  PatchPlan p;
  if (!choose(a, &BM, &p)) return (int)hipErrorInvalidConfiguration;
  const int fn = (p.NT + 3) / 4;
  if (fn <= 1) return launch_vw<64, 1>(a, p, s);
  if (fn <= 2) return launch_vw<64, 2>(a, p, s);
  return launch_vw<64, 4>(a, p, s);
}

}  // namespace ox
