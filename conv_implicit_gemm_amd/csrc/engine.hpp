// engine.hpp -- the MFMA tile engine for gfx950.
//
// One kernel template computes every dense contraction of the library:
// batched MatMul and Gemm, the 1x1 convolution and the implicit-GEMM
// convolution ("OxiONNX 0.1.7 Released", Technical Deep Dive item 2, picks
// among these three per shape; the implicit GEMM replaces the im2col + GEMM
// of tensorforge's Conv milestone M3 without materialising im2col).
//
//   out[r][c] = epilogue( sum_k L[r][k] * R[k][c] )
//
// Block: 256 threads = 4 wave64s in a 2x2 grid, block tile BM x BN, each wave
// a (BM/2) x (BN/2) tile of 16x16 MFMA blocks.  K advances in "K-units" of
// 64 bytes per row (32 bf16, 16 fp32 or 64 int8), the depth of one
// v_mfma_f32_16x16x32_bf16 / i32_16x16x64_i8 and of four f32_16x16x4f32.
//
// Both operands are staged in LDS K-contiguous per row/column, so that each
// lane's MFMA fragment (16 consecutive bytes of K for one row or column) is a
// single 128-bit LDS read.  Operands stored K-strided in memory (a [K, cols]
// matrix, an NCHW image) are transposed on the way in: a thread gathers one
// column's chunk of K with loads that are coalesced across the wave (lanes
// take consecutive columns) and writes it to LDS as one 128-bit store.
// Rows are padded by 16 bytes, which keeps both the 128-bit reads and the
// column-gather writes free of LDS bank conflicts.
//
// Pipeline: global -> registers for stage s+1 is issued before the MFMAs of
// stage s, registers -> LDS after them, one barrier per stage (double buffer).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>

#include "ox_internal.h"

namespace ox {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// The chip's 256 CUs sit in 8 XCDs, each with its own L2; consecutive block
// ids are dispatched round-robin over the XCDs.  xcd_tile maps a block id to
// a logical tile so that each XCD runs one contiguous range of the logical
// order: blocks that share an operand tile (same weight rows) then hit the
// same L2.  A bijection on [0, total) for any total.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int q = total / kXcds, r = total - q * kXcds;
  const int x = b % kXcds, local = b / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}):
// a loop unrolled at compile time whose index can select registers and
// template arguments.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// n / f.d for 0 <= n < 2^31 (see make_fastdiv)
// (umulhi(n, mul) < n, so the sum stays below 2n < 2^32: 32-bit arithmetic)
__device__ __forceinline__ int fdiv(const FastDiv& f, int n) {
  const uint32_t hi = __umulhi((uint32_t)n, f.mul);
  return (int)((hi + (uint32_t)n) >> f.shr);
}

// n / d for 0 <= n < 2^22, 1 <= d < 2^22, d not fixed for the launch: the
// single-precision product n * rcp(d) (v_rcp_f32 within 1 ulp, one more
// rounding) is within 1.5 * 2^-23 * n/d < 0.75 of n / d, so its truncation
// is off by at most one either way, which one remainder test each way
// corrects (a handful of instructions instead of the generic 32-bit
// division sequence; q * d stays below n + d, no overflow).
__device__ __forceinline__ int div_small(int n, int d) {
  int q = (int)((float)n * __builtin_amdgcn_rcpf((float)d));
  const int r = n - q * d;
  q += (r >= d) - (r < 0);
  return q;
}

// One v_mfma_f32_32x32x16_bf16: c[32x32] += a[32x16] * b[16x32].  Lane l
// supplies row (a) / column (b) l%32 with k = 8*(l/32) .. 8*(l/32)+7 as 8
// bf16 in one 128-bit register quad; accumulator element i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ void mma32(f32x16_t& c, u32x4_t a, u32x4_t b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                              __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int DT> struct Traits;
template <> struct Traits<DT_F32> {
  typedef float T;
  typedef f32x4_t Acc;
  enum { EPC = 4 };           // elements per 16-byte chunk
};
template <> struct Traits<DT_BF16> {
  typedef uint16_t T;         // raw bfloat16 bits
  typedef f32x4_t Acc;
  enum { EPC = 8 };
};
template <> struct Traits<DT_I8> {
  typedef int8_t T;
  typedef i32x4_t Acc;
  enum { EPC = 16 };
};

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (low half = lo), round to nearest even, in
// one gfx950 v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <typename T, int N>
__device__ __forceinline__ u32x4_t pack16(const T (&e)[N]) {
  static_assert(sizeof(T) * N == 16, "a chunk is 16 bytes");
  u32x4_t r;
  __builtin_memcpy(&r, e, 16);
  return r;
}

// ------------------------------------------------------------------- MFMA --

template <int DT> struct Mma;
template <> struct Mma<DT_F32> {
  __device__ __forceinline__ static void run(f32x4_t& c, u32x4_t a, u32x4_t b) {
    // four K=4 steps; lane group g holds k = 4g..4g+3 of the 16-k unit, and
    // step i takes component i from A and B alike.
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
  }
};
template <> struct Mma<DT_BF16> {
  __device__ __forceinline__ static void run(f32x4_t& c, u32x4_t a, u32x4_t b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<DT_I8> {
  __device__ __forceinline__ static void run(i32x4_t& c, u32x4_t a, u32x4_t b) {
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                              __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
  }
};

// ------------------------------------------------------------ activations --

__device__ __forceinline__ float apply_act(int act, float v) {
  switch (act) {
    case ACT_RELU: return fmaxf(v, 0.0f);
    case ACT_RELU6: return fminf(fmaxf(v, 0.0f), 6.0f);
    case ACT_GELU: return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    default: return v;
  }
}

// The same activations with the choice made at compile time: an epilogue
// that runs one per element must not carry a switch (and the GELU code) per
// element.  with_act(act, f) calls f(std::integral_constant<int, ACT>{}) for
// the runtime act, so the body is compiled once per activation.
template <int ACT>
__device__ __forceinline__ float act_c(float v) {
  if constexpr (ACT == ACT_RELU) return fmaxf(v, 0.0f);
  else if constexpr (ACT == ACT_RELU6) return __builtin_amdgcn_fmed3f(v, 0.0f, 6.0f);  // one v_med3_f32
  else if constexpr (ACT == ACT_GELU) return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
  else return v;
}

template <typename F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(std::integral_constant<int, ACT_RELU>{}); break;
    case ACT_RELU6: f(std::integral_constant<int, ACT_RELU6>{}); break;
    case ACT_GELU: f(std::integral_constant<int, ACT_GELU>{}); break;
    default: f(std::integral_constant<int, ACT_NONE>{}); break;
  }
}

// Static int8 requantisation: round half to even in fp64 (rint), add the
// output zero point, saturate.  mult is the host-computed fp64 multiplier.
__device__ __forceinline__ int8_t requant(int acc, double mult, int yzp) {
  double r = rint((double)acc * mult) + (double)yzp;
  r = fmin(fmax(r, -128.0), 127.0);
  return (int8_t)(int)r;
}

struct I8View {
  const double* mult;
  const int32_t* bias;
  const int32_t* wzp;   // per-channel weight zero points
  int xzp, yzp;         // zero points of the int8 view (a uint8 one minus 128)
  uint32_t xm;          // 0x80808080 for uint8 activations (their int8 view), else 0
  int ym;               // 0x80 for uint8 outputs, else 0
  bool wz;              // some weight zero point is nonzero
  __device__ __forceinline__ void init(const void* p) {
    const Int8Header* h = (const Int8Header*)p;
    xzp = h->x_zp;
    yzp = h->y_zp;
    const int f = h->flags;
    xm = (f & kI8XUnsigned) ? 0x80808080u : 0u;
    ym = (f & kI8YUnsigned) ? 0x80 : 0;
    wz = (f & kI8WZp) != 0;
    mult = (const double*)((const char*)p + sizeof(Int8Header));
    bias = (const int32_t*)((const char*)p + sizeof(Int8Header) + 8 * h->M);
    wzp = bias + h->M;
  }
  // requantised output byte (a uint8 output is its int8 view with the top bit flipped)
  __device__ __forceinline__ int8_t out(int acc, int ch) const {
    return (int8_t)(requant(acc, mult[ch], yzp) ^ ym);
  }
};

// FLIP (int8 only): a uint8 operand is written to LDS in its int8 view, u -
// 128 (the top bit of every byte flipped).  The flip is applied as a chunk is
// stored, not as it is loaded, so the loads stay in flight across the MMAs;
// zeros a loader supplied past K become -128 (they meet zero weights).
template <int DT, bool FLIP>
__device__ __forceinline__ u32x4_t flip_chunk(const u32x4_t& v) {
  if constexpr (DT == DT_I8 && FLIP) return v ^ 0x80808080u;
  else return v;
}

// sum of the sixteen int8 values of a 16-byte fragment, added to s
__device__ __forceinline__ int sum16_i8(const u32x4_t& v, int s) {
  s = __builtin_amdgcn_sdot4((int)v[0], 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4((int)v[1], 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4((int)v[2], 0x01010101, s, false);
  return __builtin_amdgcn_sdot4((int)v[3], 0x01010101, s, false);
}

// ---------------------------------------------------------------- loaders --
//
// Each loader owns one operand's tile for this block.  load() fetches the
// stage starting at k0 into registers, store() writes them to the LDS stage.
// LDS layout: row (or column) i of the tile at i*ROWB bytes, chunk ch (16
// bytes, EPC consecutive k) at ch*16 within the row.

template <int BKU> struct Lds {
  enum { ROWB = BKU * 64 + 16, CPR = 4 * BKU };
};

// Operand stored K-contiguous: [rows, K] with row stride ld.
template <int DT, int BROWS, int BKU, bool FLIP = false>
struct LoadRowK {
  typedef typename Traits<DT>::T T;
  enum { EPC = Traits<DT>::EPC, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         TOTAL = BROWS * CPR, NCH = (TOTAL + kThreads - 1) / kThreads };
  const T* base;
  int64_t ld;
  int nrows, K;
  bool vec;
  u32x4_t r[NCH];

  __device__ __forceinline__ void init(const T* p, int64_t ld_, int row0, int rows, int K_, bool vec_) {
    base = p + (int64_t)row0 * ld_;
    ld = ld_;
    nrows = rows - row0;
    K = K_;
    vec = vec_;
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q / CPR, ch = q % CPR;
      const int k = k0 + ch * EPC;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if ((TOTAL % kThreads == 0 || q < TOTAL) && row < nrows) {
        const T* src = base + (int64_t)row * ld + k;
        if (vec && k + EPC <= K) {
          v = *(const u32x4_t*)src;
        } else {
          T e[EPC];
#pragma unroll
          for (int j = 0; j < EPC; ++j) e[j] = (k + j < K) ? src[j] : (T)0;
          v = pack16(e);
        }
      }
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + i * kThreads;
      if (TOTAL % kThreads == 0 || q < TOTAL)
        *(u32x4_t*)(lds + (q / CPR) * ROWB + (q % CPR) * 16) = flip_chunk<DT, FLIP>(r[i]);
    }
  }
};

// Operand stored K-strided: element k of this thread's column at
// colbase[k*ld].  The thread keeps one column (tid % BCOLS) for the whole
// kernel and gathers whole chunks of K for it.
template <int DT, int BCOLS, int BKU, bool FLIP = false>
struct LoadColK {
  typedef typename Traits<DT>::T T;
  enum { EPC = Traits<DT>::EPC, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         STEP = kThreads / BCOLS,                       // chunk stride per thread
         NCH = (CPR + STEP - 1) / STEP };
  static_assert(kThreads % BCOLS == 0, "columns must divide the block");
  const T* colbase;
  int64_t ld;
  int K;
  bool valid;
  u32x4_t r[NCH];

  __device__ __forceinline__ void init_col(const T* cb, bool ok, int64_t ld_, int K_) {
    colbase = cb;
    valid = ok;
    ld = ld_;
    K = K_;
  }
  __device__ __forceinline__ void load(int k0) {
    const int ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      const int k = k0 + ch * EPC;
      T e[EPC];
#pragma unroll
      for (int j = 0; j < EPC; ++j)
        e[j] = (valid && (CPR % STEP == 0 || ch < CPR) && k + j < K) ? colbase[(int64_t)(k + j) * ld] : (T)0;
      r[i] = pack16(e);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int col = threadIdx.x % BCOLS, ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      if (CPR % STEP == 0 || ch < CPR) *(u32x4_t*)(lds + col * ROWB + ch * 16) = flip_chunk<DT, FLIP>(r[i]);
    }
  }
};

// Branch-free loaders for the pipelined K loop.  They read through raw
// buffers, where an offset with bit 31 set (kPastK) returns zeros: rows or
// columns past the operand and k past K cost no branch, so the loads of
// several stages can stay in flight behind one another.  Callers guarantee
// that every byte offset they form from the block's base stays below 2^31.
constexpr uint32_t kPastK = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7FFFFFFF, 0x00020000);
}

// bf16 bias of channel m as fp32: 0 where there is no bias or m >= M.  A raw
// buffer load (a buffer of 0 bytes when bias is null), so no branch makes
// later loads wait for it.
__device__ __forceinline__ float bias_bf16_at(const void* bias, int M, int m) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(bias), (short)0, bias ? M * 2 : 0, 0x00020000);
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, m < M ? (uint32_t)m * 2u : kPastK, 0, 0));
}

// Second pass of split-K: sum[k] = ((p_0[k] + p_1[k]) + ...) + p_{S-1}[k], in
// slice order, slice s at src + s * stride float4 values and its value k at
// [k * kstride].  The loads of G slices go out together (a slice index past S
// re-reads the last slice, whose value is then not added), so up to G slices
// cost one round trip.
template <int PER>
__device__ __forceinline__ void add_slices(const f32x4_t* src, int64_t stride, int kstride, int S,
                                           f32x4_t (&sum)[PER]) {
  constexpr int G = PER <= 2 ? 8 : 4;
  for (int s0 = 0; s0 < S; s0 += G) {
    f32x4_t v[G][PER];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const f32x4_t* p = src + (int64_t)min(s0 + j, S - 1) * stride;
#pragma unroll
      for (int k = 0; k < PER; ++k) v[j][k] = p[k * kstride];
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first add
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int k = 0; k < PER; ++k) sum[k] = s0 + j < S ? sum[k] + v[j][k] : sum[k];
  }
}

// [rows, K] operand, row stride ld, K a multiple of EPC and rows 16-byte
// aligned (a chunk is all inside K or all past it).
template <int DT, int BROWS, int BKU, bool FLIP = false>
struct LoadRowKB {
  typedef typename Traits<DT>::T T;
  enum { EPC = Traits<DT>::EPC, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         TOTAL = BROWS * CPR, NCH = (TOTAL + kThreads - 1) / kThreads };
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo[NCH];     // chunk i's byte offset in stage 0, or kPastK
  int K;
  u32x4_t r[NCH];

  __device__ __forceinline__ void init(const T* p, int64_t ld, int row0, int rows, int K_) {
    rs = operand_rsrc(p + (int64_t)row0 * ld);
    K = K_;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q / CPR, ch = q % CPR;
      const bool ok = (TOTAL % kThreads == 0 || q < TOTAL) && row < rows - row0;
      vo[i] = ok ? (uint32_t)(row * ld * (int64_t)sizeof(T)) + ch * 16 : kPastK;
    }
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = (threadIdx.x + i * kThreads) % CPR;
      const uint32_t off = k0 + ch * EPC < K ? vo[i] : kPastK;
      r[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs, off, k0 * (int)sizeof(T), 0));
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + i * kThreads;
      if (TOTAL % kThreads == 0 || q < TOTAL)
        *(u32x4_t*)(lds + (q / CPR) * ROWB + (q % CPR) * 16) = flip_chunk<DT, FLIP>(r[i]);
    }
  }
};

// [K, cols] fp32 operand, row stride ld: the thread keeps column tid % BCOLS
// and gathers the 4 consecutive k of a chunk with one load each.  (Narrower
// elements would need widening in registers whose loads are still in
// flight, which forces early waits: those take LoadColK.)
template <int DT, int BCOLS, int BKU, bool FLIP = false>
struct LoadColKB {
  typedef typename Traits<DT>::T T;
  static_assert(sizeof(T) == 4, "fp32 columns only");
  enum { EPC = Traits<DT>::EPC, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         STEP = kThreads / BCOLS, NCH = (CPR + STEP - 1) / STEP };
  static_assert(kThreads % BCOLS == 0, "columns must divide the block");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo;          // this column's byte offset at k = 0
  uint32_t ldb;         // row stride in bytes
  int K;
  bool valid;
  u32x4_t r[NCH];

  __device__ __forceinline__ void init(const T* p, int64_t ld, int col0, int cols, int K_) {
    rs = operand_rsrc(p + col0);
    const int col = threadIdx.x % BCOLS;
    valid = col < cols - col0;
    vo = (uint32_t)col * 4u;
    ldb = (uint32_t)(ld * 4);
    K = K_;
  }
  // the same with this thread's column given as a byte offset from base
  // (the columns of a block need not be evenly spaced)
  __device__ __forceinline__ void init_off(const T* base, uint32_t off, bool ok, int64_t ld, int K_) {
    rs = operand_rsrc(base);
    valid = ok;
    vo = off;
    ldb = (uint32_t)(ld * 4);
    K = K_;
  }
  __device__ __forceinline__ void load(int k0) {
    const int ch0 = threadIdx.x / BCOLS;
    const int soff = k0 * (int)ldb;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = ch * 4 + j;
        const bool ok = valid && (CPR % STEP == 0 || ch < CPR) && k0 + kk < K;
        r[i][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? vo + kk * ldb : kPastK, soff, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int col = threadIdx.x % BCOLS, ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      if (CPR % STEP == 0 || ch < CPR) *(u32x4_t*)(lds + col * ROWB + ch * 16) = r[i];
    }
  }
};

// [K, cols] bf16 operand whose columns come in aligned pairs (a 1x1
// convolution's pixels, the plane even): a task is one pair of columns and
// one 8-k chunk, loaded as eight 4-byte words (one per k, both columns,
// coalesced across the lanes) and split into the two columns' 16-byte
// chunks by byte permutes when written to LDS.  The pair's byte offset from
// base is given per thread (kPastK: past the operand).
template <int BCOLS, int BKU>
struct LoadColK2B {
  enum { CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB, G = BCOLS / 2,
         TOTAL = G * CPR, NCH = (TOTAL + kThreads - 1) / kThreads };
  static_assert(BCOLS % 2 == 0 && kThreads % G == 0, "column pairs must tile the block");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo;          // this thread's column pair at k = 0, or kPastK
  uint32_t ldb;         // row stride in bytes
  int K;
  uint32_t d[NCH][8];

  __device__ __forceinline__ void init_off(const uint16_t* base, uint32_t off, bool ok, int64_t ld, int K_) {
    rs = operand_rsrc(base);
    vo = ok ? off : kPastK;
    ldb = (uint32_t)(ld * 2);
    K = K_;
  }
  __device__ __forceinline__ void load(int k0) {
    const int soff = k0 * (int)ldb;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = threadIdx.x + i * kThreads, ch = t / G;
      const bool task = TOTAL % kThreads == 0 || t < TOTAL;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = ch * 8 + e;
        const bool ok = task && vo != kPastK && k0 + kk < K;
        d[i][e] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? vo + kk * ldb : kPastK, soff, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = threadIdx.x + i * kThreads, ch = t / G, grp = t - ch * G;
      if (TOTAL % kThreads == 0 || t < TOTAL) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // half j of each word: column 2*grp + j, k = 8ch .. 8ch+7
          const uint32_t sel = j ? 0x07060302u : 0x05040100u;
          u32x4_t v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_perm(d[i][2 * q + 1], d[i][2 * q], sel);
          *(u32x4_t*)(lds + (2 * grp + j) * ROWB + ch * 16) = v;
        }
      }
    }
  }
};

// [K, cols] bf16 operand, one column per thread at a per-thread byte offset
// (a 1x1 convolution on an odd plane, where pixel pairs are not aligned):
// each element is one 2-byte load and one 2-byte LDS write, so no
// instruction touches a loaded register before the stage that stores it.
template <int BCOLS, int BKU>
struct LoadColK1B {
  enum { EPC = 8, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         STEP = kThreads / BCOLS, NCH = (CPR + STEP - 1) / STEP };
  static_assert(kThreads % BCOLS == 0, "columns must divide the block");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo;          // this column's byte offset at k = 0, or kPastK
  uint32_t ldb;         // row stride in bytes
  int K;
  uint16_t e[NCH][EPC];

  __device__ __forceinline__ void init_off(const uint16_t* base, uint32_t off, bool ok, int64_t ld, int K_) {
    rs = operand_rsrc(base);
    vo = ok ? off : kPastK;
    ldb = (uint32_t)(ld * 2);
    K = K_;
  }
  __device__ __forceinline__ void load(int k0) {
    const int ch0 = threadIdx.x / BCOLS;
    const int soff = k0 * (int)ldb;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const int kk = ch * EPC + j;
        const bool ok = vo != kPastK && (CPR % STEP == 0 || ch < CPR) && k0 + kk < K;
        e[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? vo + kk * ldb : kPastK, soff, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int col = threadIdx.x % BCOLS, ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      if (CPR % STEP == 0 || ch < CPR) {
#pragma unroll
        for (int j = 0; j < EPC; ++j) *(uint16_t*)(lds + col * ROWB + ch * 16 + j * 2) = e[i][j];
      }
    }
  }
};

// [K, cols] int8 operand whose columns come in aligned groups of four
// consecutive bytes (a 1x1 convolution's pixels, the plane a multiple of
// four): a task is one group of four columns and one 16-k chunk, loaded as
// sixteen 4-byte words (one per k, four columns each, coalesced across the
// lanes) and transposed into the four columns' 16-byte chunks by byte
// permutes when written to LDS.  Group g's byte offset from base is given
// per thread (kPastK: the group lies past the operand).
template <int BCOLS, int BKU, bool FLIP = false>
struct LoadColK4B {
  enum { CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB, G = BCOLS / 4,
         TOTAL = G * CPR, NCH = (TOTAL + kThreads - 1) / kThreads };
  static_assert(BCOLS % 4 == 0 && kThreads % G == 0, "column groups must tile the block");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo;          // this thread's column group at k = 0, or kPastK
  uint32_t ld;          // row stride in bytes
  int K;
  uint32_t d[NCH][16];

  __device__ __forceinline__ void init_off(const int8_t* base, uint32_t off, bool ok, int64_t ld_, int K_) {
    rs = operand_rsrc(base);
    vo = ok ? off : kPastK;
    ld = (uint32_t)ld_;
    K = K_;
  }
  __device__ __forceinline__ void load(int k0) {
    const int soff = k0 * (int)ld;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = threadIdx.x + i * kThreads, ch = t / G;
      const bool task = TOTAL % kThreads == 0 || t < TOTAL;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kk = ch * 16 + e;
        const bool ok = task && vo != kPastK && k0 + kk < K;
        d[i][e] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? vo + kk * ld : kPastK, soff, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = threadIdx.x + i * kThreads, ch = t / G, grp = t - ch * G;
      if (TOTAL % kThreads == 0 || t < TOTAL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // byte j of each word: column 4*grp + j, k = 16ch .. 16ch+15
          const uint32_t sel2 = (uint32_t)j | ((uint32_t)(4 + j) << 8) | 0x0c0c0000u;
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_amdgcn_perm(d[i][4 * q + 1], d[i][4 * q], sel2);
            const uint32_t hi = __builtin_amdgcn_perm(d[i][4 * q + 3], d[i][4 * q + 2], sel2);
            w[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
          *(u32x4_t*)(lds + (4 * grp + j) * ROWB + ch * 16) =
              flip_chunk<DT_I8, FLIP>(u32x4_t{w[0], w[1], w[2], w[3]});
        }
      }
    }
  }
};

// The implicit-GEMM operand of a convolution: column = one output pixel
// (img, oh, ow), k = (c, kh, kw) in the weight's own order, element =
// X[img, c, oh*sh - pt + kh*dh, ow*sw - pl + kw*dw], or `pad` outside the
// image (0 for floats; x_zp for int8, whose zero-point fold expects it).
template <int DT, int BCOLS, int BKU, bool FLIP = false>
struct LoadIm2col {
  typedef typename Traits<DT>::T T;
  enum { EPC = Traits<DT>::EPC, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         STEP = kThreads / BCOLS, NCH = (CPR + STEP - 1) / STEP };
  const T* xb;          // X + (img*C + g*cpg) * H*W
  int ih0, iw0;
  bool valid;
  int H, W, HW, kH, kW, KK, dh, dw, K;
  T pad;                // as stored in X (flipped with the rest under FLIP)
  u32x4_t r[NCH];


  __device__ __forceinline__ void load(int k0) {
    const int ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      const int k = k0 + ch * EPC;
      T e[EPC];
      if (valid && (CPR % STEP == 0 || ch < CPR) && k < K) {
        int c = k / KK;
        int rr = k - c * KK;
        int kh = rr / kW;
        int kw = rr - kh * kW;
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          T v = (T)0;
          if (k + j < K) {
            const int ih = ih0 + kh * dh, iw = iw0 + kw * dw;
            v = ((unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W) ? xb[c * HW + ih * W + iw] : pad;
          }
          e[j] = v;
          if (++kw == kW) {
            kw = 0;
            if (++kh == kH) {
              kh = 0;
              ++c;
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPC; ++j) e[j] = (T)0;
      }
      r[i] = pack16(e);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int col = threadIdx.x % BCOLS, ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      if (CPR % STEP == 0 || ch < CPR) *(u32x4_t*)(lds + col * ROWB + ch * 16) = flip_chunk<DT, FLIP>(r[i]);
    }
  }
};

// The fp32 im2col operand through a raw buffer: the thread keeps one output
// pixel (column) and computes each element's offset from its (c, kh, kw);
// taps in the padding, k past K and columns past the range read zeros
// (kPastK), so the loads carry no branch.  The chunk's first k is split
// with two small exact divisions per stage, the rest by stepping.
template <int BCOLS, int BKU>
struct LoadIm2colB {
  enum { EPC = 4, CPR = Lds<BKU>::CPR, ROWB = Lds<BKU>::ROWB,
         STEP = kThreads / BCOLS, NCH = (CPR + STEP - 1) / STEP };
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vimg;        // byte offset of this column's image (and group) plane 0
  int ih0, iw0;
  bool valid;
  int H, W, HW, kH, kW, KK, dh, dw, K;
  u32x4_t r[NCH];

  __device__ __forceinline__ void load(int k0) {
    const int ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      const int kb = k0 + ch * EPC;
      int c = div_small(kb, KK);
      int rr = kb - c * KK;
      int kh = div_small(rr, kW);
      int kw = rr - kh * kW;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const int ih = ih0 + kh * dh, iw = iw0 + kw * dw;
        const bool ok = valid && (CPR % STEP == 0 || ch < CPR) && kb + j < K &&
                        (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
        w[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, ok ? vimg + (uint32_t)((c * HW + ih * W + iw) * 4) : kPastK, 0, 0);
        if (++kw == kW) {
          kw = 0;
          if (++kh == kH) {
            kh = 0;
            ++c;
          }
        }
      }
      r[i] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int col = threadIdx.x % BCOLS, ch0 = threadIdx.x / BCOLS;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = ch0 + i * STEP;
      if (CPR % STEP == 0 || ch < CPR) *(u32x4_t*)(lds + col * ROWB + ch * 16) = r[i];
    }
  }
};

// ------------------------------------------------------------ the kernel --

template <int DT, int BM, int BN> struct WaveTile {
  enum { TM = BM / 2, TN = BN / 2, FM = TM / 16, FN = TN / 16 };
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 16x16 block");
};

// One stage's MMAs: the BKU units of the LDS stage at As / Bs.
template <int DT, int BM, int BN, int BKU, int SUMS>
__device__ __forceinline__ void engine_stage(const char* As, const char* Bs,
                                             typename Traits<DT>::Acc (&acc)[BM / 32][BN / 32],
                                             int* ks) {
  typedef WaveTile<DT, BM, BN> WT;
  enum { ROWB = Lds<BKU>::ROWB };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int u = 0; u < BKU; ++u) {
    u32x4_t a[WT::FM], b[WT::FN];
#pragma unroll
    for (int fm = 0; fm < WT::FM; ++fm)
      a[fm] = *(const u32x4_t*)(As + (wm * WT::TM + fm * 16 + lr) * ROWB + u * 64 + lg * 16);
#pragma unroll
    for (int fn = 0; fn < WT::FN; ++fn)
      b[fn] = *(const u32x4_t*)(Bs + (wn * WT::TN + fn * 16 + lr) * ROWB + u * 64 + lg * 16);
#pragma unroll
    for (int fm = 0; fm < WT::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < WT::FN; ++fn) Mma<DT>::run(acc[fm][fn], a[fm], b[fn]);
    if constexpr (SUMS == 1) {
#pragma unroll
      for (int fm = 0; fm < WT::FM; ++fm) ks[fm] = sum16_i8(a[fm], ks[fm]);
    } else if constexpr (SUMS == 2) {
#pragma unroll
      for (int fn = 0; fn < WT::FN; ++fn) ks[fn] = sum16_i8(b[fn], ks[fn]);
    }
  }
}

// The K loop shared by every problem: accumulates into acc[FM][FN].
// SUMS (int8 only): 1 also sums the int8 values of every A row this lane
// reads into ks[fm], 2 of every B column into ks[fn]: the per-row /
// per-column activation sums of the weight zero-point term.
//
// Two LDS stages alternate.  D = 1: the next stage's global loads are issued
// before this stage's MMAs and written to LDS after them, so every stage
// waits out one global-load latency.  D = 2 or 4: D register copies of each
// loader keep the loads of stages s+1 .. s+D in flight while stage s is
// multiplied (stage t lives in copy t % D), which divides that wait by D
// for D times the loader registers.  The loop body is unrolled D times so
// that every copy index is a constant; the last 2D stages issue no loads
// past the end of K.
template <int DT, int BM, int BN, int BKU, int SUMS = 0, int D = 1, class LA, class LB>
__device__ __forceinline__ void engine_mainloop(LA& la, LB& lb, int K, char* smem,
                                                typename Traits<DT>::Acc (&acc)[BM / 32][BN / 32],
                                                int* ks = nullptr) {
  static_assert(D == 1 || D == 2 || D == 4, "1, 2 or 4 stages in flight");
  enum { ROWB = Lds<BKU>::ROWB, A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB,
         KSTEP = BKU * 4 * Traits<DT>::EPC };
  const int nk = (K + KSTEP - 1) / KSTEP;
  if (nk == 0) return;

  if constexpr (D == 1) {
    la.load(0);
    lb.load(0);
    la.store(smem);
    lb.store(smem + A_BYTES);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
      char* As = smem + (s & 1) * STAGE;
      const bool more = s + 1 < nk;
      if (more) {
        la.load((s + 1) * KSTEP);
        lb.load((s + 1) * KSTEP);
      }
      engine_stage<DT, BM, BN, BKU, SUMS>(As, As + A_BYTES, acc, ks);
      if (more) {
        char* An = smem + ((s + 1) & 1) * STAGE;
        la.store(An);
        lb.store(An + A_BYTES);
      }
      __syncthreads();
    }
  } else {
    LA pa[D];
    LB pb[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      pa[d] = la;
      pb[d] = lb;
    }
    // stages 0 .. D-1 in flight; stage 0 to LDS; stage D into copy 0
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < nk) {
        pa[d].load(d * KSTEP);
        pb[d].load(d * KSTEP);
      }
    pa[0].store(smem);
    pb[0].store(smem + A_BYTES);
    if (D < nk) {
      pa[0].load(D * KSTEP);
      pb[0].load(D * KSTEP);
    }
    __syncthreads();
    // One stage s (s % D == d): multiply it, write stage s+1 (copy (d+1)%D)
    // to the other LDS stage, refill that copy with stage s+1+D.  TAIL:
    // stage s+1 or s+1+D may not exist (the main loop knows they do, so its
    // loads are unconditional and the counter waits stay exact).
    auto step = [&](auto dk, auto tk, int s) {
      constexpr int d = decltype(dk)::value, nd = (d + 1) % D;
      constexpr bool TAIL = decltype(tk)::value;
      // keep each stage's work in its stage: hoisted uses of a loaded
      // register would wait for loads that are meant to stay in flight
      __builtin_amdgcn_sched_barrier(0);
      const char* As = smem + (d & 1) * STAGE;
      engine_stage<DT, BM, BN, BKU, SUMS>(As, As + A_BYTES, acc, ks);
      if (!TAIL || s + 1 < nk) {
        char* An = smem + ((d + 1) & 1) * STAGE;
        pa[nd].store(An);
        pb[nd].store(An + A_BYTES);
        if (!TAIL || s + 1 + D < nk) {
          pa[nd].load((s + 1 + D) * KSTEP);
          pb[nd].load((s + 1 + D) * KSTEP);
        }
      }
      __syncthreads();
    };
    int s0 = 0;
    // every stage of this loop has a successor and refills its copy
    for (; s0 + 2 * D < nk; s0 += D) {
      static_for<D>([&](auto dk) { step(dk, std::false_type{}, s0 + decltype(dk)::value); });
    }
    // the last stages: at most 2D
    static_for<2 * D>([&](auto dk) {
      constexpr int d = decltype(dk)::value;
      const int s = s0 + d;
      if (s < nk) step(std::integral_constant<int, d % D>{}, std::true_type{}, s);
    });
  }
}

// Completes the sums of engine_mainloop<SUMS> (each lane holds a quarter of
// the k range of one row or column) and writes them to S[row_in_tile]
// (SUMS 1) or S[col_in_tile] (SUMS 2) in LDS; the caller synchronises.
template <int DT, int BM, int BN, int SUMS>
__device__ __forceinline__ void ksums_to_lds(int* ks, int* S) {
  typedef WaveTile<DT, BM, BN> WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int NF = SUMS == 1 ? WT::FM : WT::FN;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int v = ks[f];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lg == 0) {
      if constexpr (SUMS == 1) {
        if (wn == 0) S[wm * WT::TM + f * 16 + lr] = v;
      } else {
        if (wm == 0) S[wn * WT::TN + f * 16 + lr] = v;
      }
    }
  }
}

// Calls f(row_in_tile, col_in_tile, value) for each of this lane's results.
// MFMA 16x16 output layout: lane l holds rows 4*(l/16)+i (i = 0..3) of column
// l%16 of its 16x16 block.
template <int BM, int BN, typename Acc, class F>
__device__ __forceinline__ void for_each_result(const Acc (&acc)[BM / 32][BN / 32], F&& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int fm = 0; fm < BM / 32; ++fm)
#pragma unroll
    for (int fn = 0; fn < BN / 32; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f(wm * (BM / 2) + fm * 16 + lg * 4 + i, wn * (BN / 2) + fn * 16 + lr, acc[fm][fn][i]);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone): every vector memory
// operation issued so far has completed.  Epilogues call it once their
// per-channel parameters are in registers and before their first store: the
// counter also counts stores, and a use of a loaded register behind a branch
// would otherwise be preceded by a wait for every earlier store as well.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Writes a BM x BN tile of a row-major output through LDS: put(E, EROW)
// stores each of this lane's results at E[row_in_tile * EROW + col_in_tile]
// (E = smem + OFF bytes), then each thread copies 16-byte pieces of the
// rows to Y (row0, col0: the tile's origin; rows / cols: Y's extent).  The
// caller checks that the staging area fits, that Y and its row stride keep
// every piece 16-byte aligned and that cols is a multiple of a piece, and
// that LDS is free (every wave is past its last read of the operands).
template <typename Y_T, int BM, int BN, int OFF, class Put>
__device__ __forceinline__ void store_tile_rows(Y_T* Y, int64_t ldy, int row0, int col0, int rows, int cols,
                                                char* smem, Put&& put) {
  constexpr int V = 16 / (int)sizeof(Y_T), EROW = BN + V, PR = BN / V;
  Y_T* E = (Y_T*)(smem + OFF);
  put(E, EROW);
  __syncthreads();
#pragma unroll
  for (int it = threadIdx.x; it < BM * PR; it += kThreads) {
    const int r = it / PR, pc = it - r * PR;
    const int row = row0 + r, col = col0 + pc * V;
    if (row < rows && col < cols)
      *(u32x4_t*)(Y + (int64_t)row * ldy + col) = *(const u32x4_t*)(E + r * EROW + pc * V);
  }
}
template <typename Y_T, int BM, int BN>
constexpr int stage_rows_bytes() { return BM * (BN + 16 / (int)sizeof(Y_T)) * (int)sizeof(Y_T); }
// whether Y (this batch's matrix) takes store_tile_rows
template <typename Y_T>
__device__ __forceinline__ bool rows_vec_ok(const Y_T* Y, int64_t ldy, int cols) {
  constexpr int V = 16 / (int)sizeof(Y_T);
  return ((uintptr_t)Y) % 16 == 0 && ldy % V == 0 && cols % V == 0;
}

// As for_each_result, with the lane's column fragment fn passed first: the
// lane's columns are lane_col<BN>(fn), fn < BN/32, so that per-column values
// can be read into registers before the first store (loads after stores
// through possibly aliasing pointers would each wait for those stores).
template <int BN>
__device__ __forceinline__ int lane_col(int fn) {
  return ((threadIdx.x >> 6) & 1) * (BN / 2) + fn * 16 + (threadIdx.x & 15);
}
// the lane's row in the tile for row fragment fm, register i
template <int BM>
__device__ __forceinline__ int lane_row(int fm, int i) {
  return (threadIdx.x >> 7) * (BM / 2) + fm * 16 + ((threadIdx.x & 63) >> 4) * 4 + i;
}
// f(fm, fn, i, row_in_tile, col_in_tile, value) for each of this lane's results
template <int BM, int BN, typename Acc, class F>
__device__ __forceinline__ void for_each_result_idx(const Acc (&acc)[BM / 32][BN / 32], F&& f) {
#pragma unroll
  for (int fm = 0; fm < BM / 32; ++fm)
#pragma unroll
    for (int fn = 0; fn < BN / 32; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) f(fm, fn, i, lane_row<BM>(fm, i), lane_col<BN>(fn), acc[fm][fn][i]);
}
template <int BM, int BN, typename Acc, class F>
__device__ __forceinline__ void for_each_result_fn(const Acc (&acc)[BM / 32][BN / 32], F&& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int fm = 0; fm < BM / 32; ++fm)
#pragma unroll
    for (int fn = 0; fn < BN / 32; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f(fn, wm * (BM / 2) + fm * 16 + lg * 4 + i, wn * (BN / 2) + fn * 16 + lr, acc[fm][fn][i]);
}

}  // namespace ox
