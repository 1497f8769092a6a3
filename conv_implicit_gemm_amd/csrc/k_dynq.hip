// k_dynq.hip -- dynamic per-tensor quantisation of fp32 activations to uint8
// (ONNX DynamicQuantizeLinear, the first node of a dynamically quantised
// MatMulInteger / ConvInteger graph):
//   lo = min(0, min x), hi = max(0, max x)       (the range always holds 0)
//   y_scale = (hi - lo) / 255                     (fp32)
//   y_zp    = rint(clamp(0 - lo / y_scale, 0, 255))
//   y       = clamp(rint(x / y_scale) + y_zp, 0, 255)
// all in fp32 with correctly rounded division and round half to even; an
// all-zero tensor gives y_scale = 0, y_zp = 0 and y = 0.
//
// Two launches on one stream: per-block partial minima / maxima into the
// caller's workspace (at most 256 blocks), then the quantising pass, whose
// blocks each finish the range from those partials (block 0 writes y_scale
// and y_zp).  Both passes over x read 16-byte vectors (grid-stride) when x is
// 16-byte aligned and y 4-byte aligned; a scalar loop takes the rest.
// Memory-bound: 9 bytes per element move (x twice, y once).
#include <cmath>

#include "engine.hpp"

namespace ox {

namespace {

constexpr int kDqMaxPartials = 256;   // blocks of the range pass (one partial each)
constexpr int kDqMaxBlocks = 1024;    // blocks of the quantising pass

__device__ __forceinline__ void block_minmax(float& lo, float& hi, float* s_lo, float* s_hi) {
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  __syncthreads();
  lo = s_lo[0];
  hi = s_hi[0];
  for (int w = 1; w < kThreads / 64; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
}

__global__ __launch_bounds__(kThreads) void dq_minmax(const float* X, int64_t n, bool vec,
                                                      float* part) {
  __shared__ float s_lo[kThreads / 64], s_hi[kThreads / 64];
  float lo = 0.0f, hi = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    const f32x4_t* X4 = (const f32x4_t*)X;
    for (int64_t i = t0; i < n4; i += stride) {
      const f32x4_t v = X4[i];
      lo = fminf(fminf(lo, v[0]), fminf(v[1], fminf(v[2], v[3])));
      hi = fmaxf(fmaxf(hi, v[0]), fmaxf(v[1], fmaxf(v[2], v[3])));
    }
    done = n4 * 4;
  }
  for (int64_t i = done + t0; i < n; i += stride) {
    lo = fminf(lo, X[i]);
    hi = fmaxf(hi, X[i]);
  }
  block_minmax(lo, hi, s_lo, s_hi);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = lo;
    part[2 * blockIdx.x + 1] = hi;
  }
}

__device__ __forceinline__ uint32_t dq_one(float x, float scale, float zp) {
  if (!(scale > 0.0f)) return 0u;
  return (uint32_t)(int)fminf(fmaxf(rintf(x / scale) + zp, 0.0f), 255.0f);
}

// Every block first finishes the range from the nb partials (a few KB, read
// from L2; the same exact min / max in every block) and derives y_scale and
// y_zp; block 0 writes them out.
__global__ __launch_bounds__(kThreads) void dq_quant(const float* X, int64_t n, bool vec,
                                                     const float* part, int nb, float* y_scale,
                                                     uint8_t* y_zp, uint8_t* Y) {
  __shared__ float s_lo[kThreads / 64], s_hi[kThreads / 64];
  float lo = 0.0f, hi = 0.0f;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    lo = fminf(lo, part[2 * i]);
    hi = fmaxf(hi, part[2 * i + 1]);
  }
  block_minmax(lo, hi, s_lo, s_hi);
  const float scale = (hi - lo) / 255.0f;
  float zp = 0.0f;
  if (scale > 0.0f) zp = rintf(fminf(fmaxf(0.0f - lo / scale, 0.0f), 255.0f));
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *y_scale = scale;
    *y_zp = (uint8_t)(int)zp;
  }
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    const f32x4_t* X4 = (const f32x4_t*)X;
    uint32_t* Y4 = (uint32_t*)Y;
    for (int64_t i = t0; i < n4; i += stride) {
      const f32x4_t v = X4[i];
      Y4[i] = dq_one(v[0], scale, zp) | (dq_one(v[1], scale, zp) << 8) |
              (dq_one(v[2], scale, zp) << 16) | (dq_one(v[3], scale, zp) << 24);
    }
    done = n4 * 4;
  }
  for (int64_t i = done + t0; i < n; i += stride) Y[i] = (uint8_t)dq_one(X[i], scale, zp);
}

int dq_blocks(int64_t n, int cap) {
  const int64_t per = (int64_t)kThreads * 16;      // 16 elements per thread and pass at least
  return (int)std::max<int64_t>(1, std::min<int64_t>(cap, (n + per - 1) / per));
}

}  // namespace

size_t dynq_workspace_bytes() { return (size_t)(2 * kDqMaxPartials) * sizeof(float); }

int launch_dynamic_quantize(int64_t n, const float* X, uint8_t* Y, float* y_scale, uint8_t* y_zp,
                            void* ws, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  float* part = (float*)ws;
  const bool vec = ((uintptr_t)X % 16) == 0 && ((uintptr_t)Y % 4) == 0;
  const int nb = dq_blocks(n, kDqMaxPartials);
  hipLaunchKernelGGL(dq_minmax, dim3(nb), dim3(kThreads), 0, s, X, n, vec, part);
  hipLaunchKernelGGL(dq_quant, dim3(dq_blocks(n, kDqMaxBlocks)), dim3(kThreads), 0, s, X, n, vec,
                     (const float*)part, nb, y_scale, y_zp, Y);
  return (int)hipGetLastError();
}

}  // namespace ox
