// k_gemv.hip -- Gemm with one output row (M = 1), float path.
//
//   y[j] = act(alpha * sum_k x[k] * B'[k,j] + beta * bias[j])
//
// With one row there is nothing to reuse: every weight is read once, so the
// kernel is bound by HBM and a tile engine would idle its MFMA units.
// transB (weights [N,K], the MLP layout): a block owns RB (1..8) output
// columns, i.e. RB weight rows, and its four waves split K in quarters; the
// lanes of a wave sweep their quarter in 16-byte chunks (one chunk of x serves
// all RB rows) with two iterations of loads in flight, so that a launch of
// N / RB >= 512 blocks keeps the whole weight matrix streaming.  Each row's
// partial sums are reduced across the wave with shuffles and across the four
// waves through LDS, always in the same order, so the result is bitwise
// repeatable.  Without transB (weights [K,N]) each lane owns one column and
// the four waves split K, then combine their partial sums through LDS in a
// fixed order.
#include "engine.hpp"

namespace ox {

namespace {

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

// weights [N, K] (K contiguous): block = RB rows x K, wave w = K quarter w
template <typename T, int RB>
__global__ __launch_bounds__(kThreads) void gemv_nk_kernel(const GemmArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  __shared__ float part[kThreads / 64][RB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = blockIdx.x * RB;
  const T* x = (const T*)a.L;
  const T* Wt = (const T*)a.R;
  const int K = a.K;
  float s[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) s[r] = 0.f;
  const T* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) wrow[r] = Wt + (int64_t)min(j0 + r, a.cols - 1) * a.ldr;   // clamped: row j0+r may not exist
  if (a.r_vec && a.l_vec) {
    // this wave's quarter of the 16-byte chunks
    const int nch = K / EPC;
    const int q = (nch + 3) / 4;
    const int cb = wave * q, ce = min(nch, cb + q);
    int ch = cb + lane;
    for (; ch + 64 < ce; ch += 128) {
      u32x4_t xr0 = *(const u32x4_t*)(x + ch * EPC), xr1 = *(const u32x4_t*)(x + (ch + 64) * EPC);
      u32x4_t wr0[RB], wr1[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        wr0[r] = *(const u32x4_t*)(wrow[r] + ch * EPC);
        wr1[r] = *(const u32x4_t*)(wrow[r] + (ch + 64) * EPC);
      }
      float xf0[EPC], xf1[EPC];
      chunk_to_f32<T>(xr0, xf0);
      chunk_to_f32<T>(xr1, xf1);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float wf0[EPC], wf1[EPC];
        chunk_to_f32<T>(wr0[r], wf0);
        chunk_to_f32<T>(wr1[r], wf1);
#pragma unroll
        for (int e = 0; e < EPC; ++e) s[r] += xf0[e] * wf0[e];
#pragma unroll
        for (int e = 0; e < EPC; ++e) s[r] += xf1[e] * wf1[e];
      }
    }
    if (ch < ce) {
      float xf[EPC];
      chunk_to_f32<T>(*(const u32x4_t*)(x + ch * EPC), xf);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float wf[EPC];
        chunk_to_f32<T>(*(const u32x4_t*)(wrow[r] + ch * EPC), wf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) s[r] += xf[e] * wf[e];
      }
    }
    // the elements past the last whole chunk: wave 3
    if (wave == 3)
      for (int k = nch * EPC + lane; k < K; k += 64) {
        const float xv = to_f32(x[k]);
#pragma unroll
        for (int r = 0; r < RB; ++r) s[r] += xv * to_f32(wrow[r][k]);
      }
  } else {
    const int q = (K + 3) / 4;
    const int kb = wave * q, ke = min(K, kb + q);
    for (int k = kb + lane; k < ke; k += 64) {
      const float xv = to_f32(x[k]);
#pragma unroll
      for (int r = 0; r < RB; ++r) s[r] += xv * to_f32(wrow[r][k]);
    }
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) s[r] = wave_sum(s[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) part[wave][r] = s[r];
  }
  __syncthreads();
  if (threadIdx.x < RB && j0 + (int)threadIdx.x < a.cols) {
    const int r = threadIdx.x;
    finish<T>(a, j0 + r, ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r]);
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

template <typename T, int RB>
void launch_nk(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemv_nk_kernel<T, RB>), dim3((a.cols + RB - 1) / RB), dim3(kThreads), 0, s, a);
}

template <typename T>
int launch_t(const GemmArgs& a, hipStream_t s) {
  if (a.r_kmajor) {
    // rows per block: as many as keep >= 512 blocks (at most 8)
    const int rb = a.cols >= 4096 ? 8 : a.cols >= 2048 ? 4 : a.cols >= 1024 ? 2 : 1;
    if (rb == 8) launch_nk<T, 8>(a, s);
    else if (rb == 4) launch_nk<T, 4>(a, s);
    else if (rb == 2) launch_nk<T, 2>(a, s);
    else launch_nk<T, 1>(a, s);
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
