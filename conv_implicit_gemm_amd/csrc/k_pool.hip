// k_pool.hip -- the memory-bound steps beside the convolutions: inference
// BatchNormalization + activation (a BatchNorm that cannot be folded into a
// convolution, e.g. the pre-activation BN -> ReLU of a ResNet-v2 block),
// MaxPool and GlobalAveragePool (NCHW).  No MFMA: each reads its input once
// and writes its output once, so each is measured against HBM bandwidth.
#include <algorithm>
#include <cmath>

#include "engine.hpp"

namespace ox {

namespace {

// ---------------------------------------------------- BatchNorm + act ----
// Y = act((X - mean[c]) * (gamma[c] / sqrt(var[c] + eps)) + beta[c]).  The
// flat NCHW range is walked in vectors of V elements (16 bytes when the
// pointers allow and a plane holds at least V elements, so that a vector
// crosses at most one plane boundary: its elements take the channel of
// their own plane), grid-stride, two vectors per thread and step in flight;
// the last total % V elements go element by element.
template <typename T, int V, int ACT>
__global__ __launch_bounds__(kThreads) void bn_act_kernel(const PoolArgs a) {
  const T* X = (const T*)a.X;
  T* Y = (T*)a.Y;
  const int64_t nvec = a.total / V;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  auto params = [&](int c, float& sc, float& sh) {
    sc = a.gamma[c] / sqrtf(a.var[c] + a.eps);
    sh = a.beta[c] - a.mean[c] * sc;
  };
  auto one = [&](int64_t v) {
    const int64_t e0 = v * V;
    const int64_t p0 = e0 / a.HW;
    const int left = (int)(a.HW - (e0 - p0 * a.HW));      // elements of this vector in plane p0 (>= 1)
    const int c0 = (int)(p0 % a.C);
    float sc0, sh0, sc1 = 0.f, sh1 = 0.f;
    params(c0, sc0, sh0);
    if (left < V) params(c0 + 1 == a.C ? 0 : c0 + 1, sc1, sh1);
    T in[V], out[V];
    if constexpr (V * sizeof(T) == 16) {
      const u32x4_t raw = *(const u32x4_t*)(X + e0);
      __builtin_memcpy(in, &raw, 16);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) in[j] = X[e0 + j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const bool first = j < left;
      const float y = act_c<ACT>(fmaf(to_f32(in[j]), first ? sc0 : sc1, first ? sh0 : sh1));
      if constexpr (sizeof(T) == 2) out[j] = f32_to_bf16(y);
      else out[j] = y;
    }
    if constexpr (V * sizeof(T) == 16) {
      u32x4_t raw;
      __builtin_memcpy(&raw, out, 16);
      *(u32x4_t*)(Y + e0) = raw;
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) Y[e0 + j] = out[j];
    }
  };
  int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; v + stride < nvec; v += 2 * stride) {
    one(v);
    one(v + stride);
  }
  if (v < nvec) one(v);
  if (blockIdx.x == 0) {
    for (int64_t e = nvec * V + threadIdx.x; e < a.total; e += kThreads) {
      const int c = (int)((e / a.HW) % a.C);
      float sc, sh;
      params(c, sc, sh);
      const float y = act_c<ACT>(fmaf(to_f32(X[e]), sc, sh));
      if constexpr (sizeof(T) == 2) Y[e] = f32_to_bf16(y);
      else Y[e] = y;
    }
  }
}

// ------------------------------------------------------------- MaxPool ----
// One thread per output element (consecutive threads on consecutive output
// columns); the window is read straight from global memory, the neighbours'
// overlapping windows meeting in the caches.  Padding cells never win.
template <typename T>
__global__ __launch_bounds__(kThreads) void maxpool_kernel(const PoolArgs a) {
  const T* X = (const T*)a.X;
  T* Y = (T*)a.Y;
  const int64_t total = (int64_t)a.planes * a.Ho * a.Wo;
  for (int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * kThreads) {
    const int ow = (int)(o % a.Wo);
    const int oh = (int)((o / a.Wo) % a.Ho);
    const int64_t plane = o / ((int64_t)a.Wo * a.Ho);
    const T* xp = X + plane * a.H * a.W;
    float best = -INFINITY;
    for (int kh = 0; kh < a.kH; ++kh) {
      const int ih = oh * a.sh - a.pt + kh * a.dh;
      if ((unsigned)ih >= (unsigned)a.H) continue;
      for (int kw = 0; kw < a.kW; ++kw) {
        const int iw = ow * a.sw - a.pl + kw * a.dw;
        if ((unsigned)iw >= (unsigned)a.W) continue;
        best = fmaxf(best, to_f32(xp[ih * a.W + iw]));
      }
    }
    if constexpr (sizeof(T) == 2) Y[o] = f32_to_bf16(best);   // (a maximum of bf16 values is one: exact)
    else Y[o] = best;
  }
}

// -------------------------------------------------- GlobalAveragePool ----
// One wave per plane: lanes stride over the plane summing in fp32, then a
// butterfly reduction in a fixed order (the same bits every run); lane 0
// writes sum / HW.
template <typename T>
__global__ __launch_bounds__(kThreads) void gap_kernel(const PoolArgs a) {
  const T* X = (const T*)a.X;
  T* Y = (T*)a.Y;
  const int lane = threadIdx.x & 63;
  const int64_t plane = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (plane >= a.planes) return;
  const T* xp = X + plane * a.HW;
  float s = 0.f;
  for (int i = lane; i < a.HW; i += 64) s += to_f32(xp[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    const float m = s / (float)a.HW;
    if constexpr (sizeof(T) == 2) Y[plane] = f32_to_bf16(m);
    else Y[plane] = m;
  }
}

template <typename F>
void with_act_host(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(std::integral_constant<int, ACT_RELU>{}); break;
    case ACT_RELU6: f(std::integral_constant<int, ACT_RELU6>{}); break;
    case ACT_GELU: f(std::integral_constant<int, ACT_GELU>{}); break;
    default: f(std::integral_constant<int, ACT_NONE>{}); break;
  }
}

int blocks_for(int64_t items) {
  const int64_t b = (items + kThreads - 1) / kThreads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(b, 256 * 16));
}

template <typename T>
int launch_bn(const PoolArgs& a, hipStream_t s) {
  constexpr int V16 = 16 / sizeof(T);
  const bool vec = ((uintptr_t)a.X % 16 == 0) && ((uintptr_t)a.Y % 16 == 0) && a.HW >= V16;
  const int64_t nvec = vec ? a.total / V16 : a.total;
  dim3 grid(blocks_for((nvec + 1) / 2));
  with_act_host(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
    if (vec) hipLaunchKernelGGL((bn_act_kernel<T, V16, ACT>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((bn_act_kernel<T, 1, ACT>), grid, dim3(kThreads), 0, s, a);
  });
  return (int)hipGetLastError();
}

}  // namespace

int launch_bn_act(const PoolArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  return a.dt == DT_F32 ? launch_bn<float>(a, s) : launch_bn<uint16_t>(a, s);
}

int launch_maxpool(const PoolArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(blocks_for((int64_t)a.planes * a.Ho * a.Wo));
  if (a.dt == DT_F32) hipLaunchKernelGGL((maxpool_kernel<float>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((maxpool_kernel<uint16_t>), grid, dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

int launch_global_avgpool(const PoolArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid((unsigned)((a.planes + kThreads / 64 - 1) / (kThreads / 64)));
  if (a.dt == DT_F32) hipLaunchKernelGGL((gap_kernel<float>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((gap_kernel<uint16_t>), grid, dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace ox
