// k_nbits.hip -- weight-only int4 MatMul (ONNX MatMulNBits, 4 bits, blocks
// of 32 along K): Y[M,N] = A[M,K] x dequant(B)^T (+ bias), A / bias / Y bf16.
// B stays packed in HBM, as its column blocks [N][K/32][16 bytes] (element k
// of a block in byte k/2, the low nibble for even k), with an fp32 scale per
// block and an optional 4-bit zero point per block (packed two per byte,
// default 8): w = (q - zp) * scale.
//
// Decode rows (M <= 4) take a fused matrix-vector kernel (below).  Prefill:
// the MFMA tile engine runs it as a bf16 GEMM whose B operand is a loader
// that fetches 4 packed bytes (8 weights), the block's scale and zero point
// per 16-byte LDS chunk, and dequantises to bf16 (round to nearest even) as
// the chunk is written to LDS -- the prefill tiled matmul that dequantises
// each weight tile into shared memory on load.  A K stage of the engine
// (64 bf16) is two quantisation blocks.
#include "engine.hpp"

namespace ox {

namespace {

template <int BCOLS, int BKU>
struct LoadNBits {
  enum { EPC = 8, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         TOTAL = BCOLS * CPR, NCH = (TOTAL + kThreads - 1) / kThreads };
  const uint8_t* qb;      // B blocks of this tile's first column
  const float* sc;        // scales of this tile's first column
  const uint8_t* zp;      // zero points of this tile's first column (or null)
  int nblk, zstride, ncols, K;
  uint32_t q[NCH];
  float s[NCH];
  int z[NCH];

  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int col = c / CPR, ch = c % CPR;
      const int k = k0 + ch * EPC;
      uint32_t qv = 0u;
      float sv = 0.0f;
      int zv = 8;
      if ((TOTAL % kThreads == 0 || c < TOTAL) && col < ncols && k < K) {
        const int blk = k >> 5;
        qv = *(const uint32_t*)(qb + ((int64_t)col * nblk + blk) * 16 + ((k & 31) >> 1));
        sv = sc[(int64_t)col * nblk + blk];
        if (zp) zv = (zp[(int64_t)col * zstride + (blk >> 1)] >> ((blk & 1) * 4)) & 15;
      }
      q[i] = qv;
      s[i] = sv;
      z[i] = zv;
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (TOTAL % kThreads == 0 || c < TOTAL) {
        float w[EPC];
#pragma unroll
        for (int j = 0; j < EPC; ++j) w[j] = (float)((int)((q[i] >> (4 * j)) & 15u) - z[i]) * s[i];
        const u32x4_t v = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                           pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
        *(u32x4_t*)(lds + (c / CPR) * ROWB + (c % CPR) * 16) = v;
      }
    }
  }
};

template <int BM, int BN, int BKU>
__global__ __launch_bounds__(kThreads) void nbits_gemm_kernel(const NBitsArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * Lds<BKU>::ROWB];
  const int row0 = blockIdx.y * BM, col0 = blockIdx.x * BN;

  LoadRowK<DT_BF16, BM, BKU> la;
  la.init((const uint16_t*)a.A, a.lda, row0, a.M, a.K, a.a_vec);
  LoadNBits<BN, BKU> lb;
  lb.qb = a.B;
  lb.sc = a.scales;
  lb.zp = a.zp;
  lb.nblk = a.nblk;
  lb.zstride = (a.nblk + 1) / 2;
  lb.ncols = a.N - col0;
  lb.K = a.K;
  lb.qb += (int64_t)col0 * a.nblk * 16;
  lb.sc += (int64_t)col0 * a.nblk;
  if (lb.zp) lb.zp += (int64_t)col0 * lb.zstride;

  f32x4_t acc[BM / 32][BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < BN / 32; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  engine_mainloop<DT_BF16, BM, BN, BKU>(la, lb, a.K, smem, acc);

  uint16_t* Y = (uint16_t*)a.Y;
  const uint16_t* bias = (const uint16_t*)a.bias;
  // the lane's columns' biases, read before any store (a load behind a
  // store would wait for it)
  float bc[BN / 32];
#pragma unroll
  for (int fn = 0; fn < BN / 32; ++fn)
    bc[fn] = bias ? bf16_to_f32(bias[min(col0 + lane_col<BN>(fn), a.N - 1)]) : 0.0f;
  wait_vmem();
  for_each_result_fn<BM, BN>(acc, [&](int fn, int r, int c, float v) {
    const int row = row0 + r, col = col0 + c;
    if (row < a.M && col < a.N) {
      if (bias) v += bc[fn];
      Y[(int64_t)row * a.ldy + col] = f32_to_bf16(v);
    }
  });
}

// Decode: a fused matrix-vector product straight from the nibbles.  One
// wave per output column n; lane l takes blocks l, l+64, ... of that column
// (16 packed bytes = 32 weights in one 16-byte load, its scale and zero
// point) and the matching 32 activations of each of the MR rows, sums
// a * (q - zp) in fp32 per block and scales once per block; the wave's lanes
// are then added with shuffles.  Weights are not rounded to bf16 here.
template <int MR>
__global__ __launch_bounds__(kThreads) void nbits_gemv_kernel(const NBitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (n >= a.N) return;                     // whole waves; no barrier follows
  const uint8_t* qrow = a.B + (int64_t)n * a.nblk * 16;
  const float* srow = a.scales + (int64_t)n * a.nblk;
  const uint8_t* zrow = a.zp ? a.zp + (int64_t)n * ((a.nblk + 1) / 2) : nullptr;
  const uint16_t* A = (const uint16_t*)a.A;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  for (int b = lane; b < a.nblk; b += 64) {
    const u32x4_t qv = *(const u32x4_t*)(qrow + (int64_t)b * 16);
    const float sc = srow[b];
    const int z = zrow ? (zrow[b >> 1] >> ((b & 1) * 4)) & 15 : 8;
    float w[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) w[j] = (float)((int)((qv[j >> 3] >> (4 * (j & 7))) & 15u) - z);
    const int k0 = b * 32;
    const bool full = a.a_vec && k0 + 32 <= a.K;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint16_t* ar = A + (int64_t)m * a.lda + k0;
      float s = 0.0f;
      if (full) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_t av = *(const u32x4_t*)(ar + 8 * c);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            s += __uint_as_float(av[h] << 16) * w[8 * c + 2 * h];
            s += __uint_as_float(av[h] & 0xffff0000u) * w[8 * c + 2 * h + 1];
          }
        }
      } else {
        for (int j = 0; j < 32 && k0 + j < a.K; ++j) s += bf16_to_f32(ar[j]) * w[j];
      }
      acc[m] += s * sc;
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    acc[m] = v;
  }
  if (lane == 0) {
    const uint16_t* bias = (const uint16_t*)a.bias;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
    uint16_t* Y = (uint16_t*)a.Y;
#pragma unroll
    for (int m = 0; m < MR; ++m) Y[(int64_t)m * a.ldy + n] = f32_to_bf16(acc[m] + bv);
  }
}

template <int BM, int BN, int BKU>
int launch_tile(const NBitsArgs& a, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, 1);
  hipLaunchKernelGGL((nbits_gemm_kernel<BM, BN, BKU>), grid, dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

template <int MR>
int launch_gemv(const NBitsArgs& a, hipStream_t s) {
  constexpr int WPB = kThreads / 64;
  hipLaunchKernelGGL((nbits_gemv_kernel<MR>), dim3((a.N + WPB - 1) / WPB), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

bool nbits_gemv_ok(const NBitsArgs& a) { return a.M <= 4 && ((uintptr_t)a.B % 16) == 0; }

int launch_matmul_nbits(const NBitsArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // decode (up to 4 rows): the fused matrix-vector kernel, one wave per
  // output column; prefill: the tile engine, 32x32 tiles with four
  // quantisation blocks per K stage while the grid would not fill the chip
  // with 64x64 tiles (two blocks per stage)
  if (nbits_gemv_ok(a)) {
    switch (a.M) {
      case 1: return launch_gemv<1>(a, s);
      case 2: return launch_gemv<2>(a, s);
      case 3: return launch_gemv<3>(a, s);
      default: return launch_gemv<4>(a, s);
    }
  }
  const int64_t tiles64 = (int64_t)((a.N + 63) / 64) * ((a.M + 63) / 64);
  if (tiles64 < 512) return launch_tile<32, 32, 4>(a, s);
  return launch_tile<64, 64, 2>(a, s);
}

}  // namespace ox
