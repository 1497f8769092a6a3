// k_gemv.hip -- Gemm with one output row (M = 1), float path.
//
//   y[j] = act(alpha * sum_k x[k] * B'[k,j] + beta * bias[j])
//
// With one row there is nothing to reuse: every weight is read once, so the
// kernel is bound by HBM and a tile engine would idle its MFMA units.
// transB (weights [N,K], the MLP layout): each wave owns 4 output columns;
// its lanes sweep K in 16-byte chunks (one chunk of x serves all 4 rows) and
// the four partial sums are reduced across the wave with shuffles, in a fixed
// order, so the result is bitwise repeatable.  Without transB (weights [K,N])
// each lane owns one column and the four waves split K, then combine their
// partial sums through LDS in a fixed order.
#include "engine.hpp"

namespace ox {

namespace {

constexpr int kRowsPerWave = 4;

template <typename T>
__device__ __forceinline__ void chunk_to_f32(u32x4_t raw, float (&f)[16 / sizeof(T)]);
template <> __device__ __forceinline__ void chunk_to_f32<float>(u32x4_t raw, float (&f)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(raw[i]);
}
template <> __device__ __forceinline__ void chunk_to_f32<uint16_t>(u32x4_t raw, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(raw[i] << 16);
    f[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ void finish(const GemmArgs& a, int j, float s) {
  const T* bias = (const T*)a.bias;
  float o = a.alpha * s;
  if (bias) o += a.beta * to_f32(bias[j]);
  o = apply_act(a.act, o);
  if constexpr (sizeof(T) == 2) ((uint16_t*)a.Y)[j] = f32_to_bf16(o);
  else ((float*)a.Y)[j] = o;
}

// weights [N, K] (K contiguous)
template <typename T>
__global__ __launch_bounds__(kThreads) void gemv_nk_kernel(const GemmArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = (blockIdx.x * (kThreads / 64) + wave) * kRowsPerWave;
  const T* x = (const T*)a.L;
  const T* Wt = (const T*)a.R;
  const int K = a.K;
  float s[kRowsPerWave] = {0.f, 0.f, 0.f, 0.f};
  if (a.r_vec && a.l_vec) {
    const int nch = K / EPC;
    for (int ch = lane; ch < nch; ch += 64) {
      float xf[EPC];
      chunk_to_f32<T>(*(const u32x4_t*)(x + ch * EPC), xf);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int j = j0 + r;
        if (j < a.cols) {
          float wf[EPC];
          chunk_to_f32<T>(*(const u32x4_t*)(Wt + (int64_t)j * a.ldr + ch * EPC), wf);
#pragma unroll
          for (int e = 0; e < EPC; ++e) s[r] += xf[e] * wf[e];
        }
      }
    }
    for (int k = nch * EPC + lane; k < K; k += 64) {
      const float xv = to_f32(x[k]);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
        if (j0 + r < a.cols) s[r] += xv * to_f32(Wt[(int64_t)(j0 + r) * a.ldr + k]);
    }
  } else {
    for (int k = lane; k < K; k += 64) {
      const float xv = to_f32(x[k]);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
        if (j0 + r < a.cols) s[r] += xv * to_f32(Wt[(int64_t)(j0 + r) * a.ldr + k]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) s[r] = wave_sum(s[r]);
  if (lane < kRowsPerWave && j0 + lane < a.cols) {
    float v = s[0];
#pragma unroll
    for (int r = 1; r < kRowsPerWave; ++r)
      if (lane == r) v = s[r];
    finish<T>(a, j0 + lane, v);
  }
}

// weights [K, N] (N contiguous)
template <typename T>
__global__ __launch_bounds__(kThreads) void gemv_kn_kernel(const GemmArgs a) {
  __shared__ float part[kThreads / 64][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const T* x = (const T*)a.L;
  const T* Wt = (const T*)a.R;
  const int K = a.K, nw = kThreads / 64;
  const int kper = (K + nw - 1) / nw;
  const int kb = wave * kper, ke = min(K, kb + kper);
  float s = 0.f;
  if (j < a.cols)
    for (int k = kb; k < ke; ++k) s += to_f32(x[k]) * to_f32(Wt[(int64_t)k * a.ldr + j]);
  part[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && j < a.cols) {
    float v = part[0][lane];
    for (int w = 1; w < nw; ++w) v += part[w][lane];
    finish<T>(a, j, v);
  }
}

template <typename T>
int launch_t(const GemmArgs& a, hipStream_t s) {
  if (a.r_kmajor) {
    const int per_block = (kThreads / 64) * kRowsPerWave;
    dim3 grid((a.cols + per_block - 1) / per_block);
    hipLaunchKernelGGL(gemv_nk_kernel<T>, grid, dim3(kThreads), 0, s, a);
  } else {
    dim3 grid((a.cols + 63) / 64);
    hipLaunchKernelGGL(gemv_kn_kernel<T>, grid, dim3(kThreads), 0, s, a);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_gemv(const GemmArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.dt == DT_F32) return launch_t<float>(a, s);
  if (a.dt == DT_BF16) return launch_t<uint16_t>(a, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace ox
