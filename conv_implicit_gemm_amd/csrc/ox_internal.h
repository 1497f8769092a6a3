// ox_internal.h -- launch descriptions shared by the C-ABI front end
// (ox_api.cpp, host only) and the kernel translation units (*.hip).
//
// The front end validates every argument and picks a kernel variant before
// any of these structures reaches a launcher; launchers trust them.
#pragma once

#include <stdint.h>

namespace ox {

// storage types (same values as ox_dtype)
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_I8 = 2, DT_I32 = 3 };

// activations (same values as ox_act)
enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_RELU6 = 2, ACT_GELU = 3 };

// Tile shapes of the MFMA tile engine (block tile BM x BN, 4 waves in 2x2).
enum Tile : int {
  TILE_128x128 = 0,
  TILE_64x128 = 1,
  TILE_128x64 = 2,
  TILE_64x64 = 3,
  TILE_32x64 = 4,
  TILE_COUNT = 5
};

inline int tile_bm(int t) {
  static const int v[TILE_COUNT] = {128, 64, 128, 64, 32};
  return v[t];
}
inline int tile_bn(int t) {
  static const int v[TILE_COUNT] = {128, 128, 64, 64, 64};
  return v[t];
}
inline const char* tile_name(int t) {
  static const char* v[TILE_COUNT] = {"128x128", "64x128", "128x64", "64x64", "32x64"};
  return v[t];
}

// Layout of the int8 parameter block (device copy of ox_int8_prepare's
// output): a 32-byte header, then mult[M] (fp64), bias_fold[M] (int32) and
// w_zp[M] (int32).  x_zp and y_zp are the zero points as the kernels use
// them: a uint8 tensor is read as int8 after flipping its top bit (u - 128),
// so its zero point is stored minus 128.
struct Int8Header {
  int32_t magic;       // 'OXI8'
  int32_t version;     // 2
  int64_t M;
  int32_t x_zp;
  int32_t y_zp;
  int32_t flags;       // kI8XUnsigned | kI8YUnsigned | kI8WZp
  int32_t reserved;
};
static_assert(sizeof(Int8Header) == 32, "int8 header is 32 bytes");
constexpr int32_t kInt8Magic = 0x3849584F;  // "OXI8" little-endian
constexpr int32_t kI8XUnsigned = 1;         // activations are uint8
constexpr int32_t kI8YUnsigned = 2;         // requantised outputs are uint8
constexpr int32_t kI8WZp = 4;               // some weight zero point is nonzero

// A GEMM on the tile engine: rows x cols output, reduction K, batch in z.
//   out[z][r][c] = epi( sum_k L[z][r][k] * R[z][k][c] )
// L: rows operand; l_kmajor = 1 when stored [rows, K] (K contiguous, row
//    stride ldl), 0 when stored [K, rows] (rows contiguous, k stride ldl).
// R: cols operand; r_kmajor = 1 when stored [cols, K] (K contiguous, col
//    stride ldr), 0 when stored [K, cols] (cols contiguous, k stride ldr).
struct GemmArgs {
  int dt;                 // input type: DT_F32, DT_BF16 or DT_I8
  int out_dt;             // DT_F32/DT_BF16 (= dt) or DT_I8/DT_I32 for int8 input
  int rows, cols, K, batch;
  const void* L; int64_t ldl, sl; int l_kmajor;
  const void* R; int64_t ldr, sr; int r_kmajor;
  void* Y; int64_t ldy, sy;
  const void* bias;       // [cols] or null (float path)
  float alpha, beta;
  int act;
  const void* i8;         // int8 parameter block (int8 path), channel = col
  int l_vec, r_vec;       // 16-byte vector loads allowed for a K-major operand
  int tile_group;         // row tiles per group of the block -> tile order (set at launch)
};

// A convolution (NCHW) on the tile engine: rows = output channels of one
// group, cols = N*Ho*Wo output pixels, K = C/group * kH * kW, group in z.
struct ConvArgs {
  int dt;                 // DT_F32, DT_BF16 or DT_I8
  int out_dt;
  int N, C, H, W, M, kH, kW, sh, sw, pt, pl, dh, dw, group, Ho, Wo;
  const void* X;
  const void* Wt;         // [M, C/group, kH, kW]
  const void* bias;       // [M] or null (float path)
  void* Y;
  int act;
  const void* i8;         // int8 parameter block, channel = m
  int w_vec;              // weight rows allow 16-byte vector loads
  int x_vec;              // (1x1 only) pixel rows allow 16-byte loads
  int w_packed;           // Wt is in the packed tap-major layout (see ox_conv2d_pack_weights)
  void* ws;               // caller's scratch for split-K partials, or null (no split-K)
  size_t ws_bytes;        // its size
  const void* res;        // residual [N, M, Ho, Wo] of Y's type, added before the activation, or null
};

// Division by a divisor fixed for a launch (0 <= n < 2^31, 1 <= d < 2^31):
// q = (umulhi(n, mul) + n) >> shr with a 33-bit magic multiplier whose top
// bit is implicit.  Set on the host, used in kernels where a runtime
// division per element would cost more than the element's arithmetic.
struct FastDiv {
  uint32_t d, mul, shr;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.shr = 0;
  while ((1ull << f.shr) < d) ++f.shr;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << f.shr) - d)) / d + 1);
  return f;
}

// Plan of the LDS-patch 3x3 kernel (host-chosen, passed to the kernel by
// value): configuration, block band and patch geometry.
struct PatchPlan {
  int BM, WM, FN, UPT;  // channels per block, wave rows, 32-pixel tiles per wave, staging units per thread
  int TR;               // output rows per block (per image)
  int IMB;              // images per block (> 1 only when TR == Ho)
  int PR;               // patch rows per image
  int PWs;              // patch columns per stride phase
  int PWt;              // patch row length in cells (stride * PWs)
  int PW;               // patch columns used
  int NT;               // 32-pixel tiles per block
  int nrb;              // row blocks per image
  int nib;              // image blocks
  int nmb;              // output-channel blocks
  int npos;             // cells in the patch (IMB * PR * PWt)
  int VW;               // plane positions per staging unit (1, 2, 4 or 8)
  int units;            // upper bound of staging units per block
  int lds;              // bytes of LDS
  int ga, gb;           // XCD rectangles: pixel blocks in ga groups x channel blocks in gb
  int splits;           // slices of the channel chunks per tile (split-K), 1 = none
  int cps;              // chunks per slice
  float* ws;            // split-K partials (splits * tiles * BM * NT*32 floats), else null
};

// Plan of the pointwise (1x1) kernel: block configuration and launch grid.
struct PwPlan {
  int WM;     // wave rows: 64*WM output channels, 32*(4/WM)*FP pixels per block
  int FP;     // 32-pixel fragments per wave (1 or 2)
  int KC;     // input channels per chunk (32 or 64)
  int P;      // pixels per staging load (1, 2 or 4)
  int V;      // pixels per output store (1, 2, 4 or 8)
  int npb;    // pixel blocks
  int nmb;    // output-channel blocks
  int lds;    // bytes of LDS
  int bias_lds;  // of which the staged bias vector (its tail)
  int grid;   // persistent blocks (work units are strided over them)
  int splits; // slices of the channel range per tile (split-K), 1 = none
  int cps;    // chunks per slice
  float* ws;  // split-K partials (splits * tiles * BM * BN floats), else null
};

// Plan of the DMA-staged pointwise kernel (bf16 1x1 with H*W even):
// tile BP pixels x BC output channels, KC input channels per stage, S ring
// stages, WP waves along the pixels (4/WP along the channels).  The grid is
// persistent: nranges x nmb blocks, block (r, mb) computes channel block mb
// over pixel range r = [r*span, min((r+1)*span, Q)), span = kunits * unit
// pixels with unit = 64 or 128 -- in tiles of BP pixels.
struct PwdPlan {
  int BP, BC, KC, S, WP;
  int PB;                 // bytes per pixel DMA piece: 16 (H*W % 8 == 0) or 4 (H*W even)
  int V;                  // pixels per output store (8, 4, 2 or 1; H*W % V == 0)
  int nmb;                // channel blocks
  int nranges;            // pixel ranges
  int grid;               // nranges * nmb blocks
  int span;               // pixels per range (a multiple of 64)
  int Q;                  // pixels of the batch (N * H * W)
  FastDiv hw;             // division by H * W
  uint32_t x_bytes, w_bytes;   // buffer ranges of X and W
  int lds;                // bytes of LDS
};

// The static device scratch array (k_static_scratch.hip): its size, and its
// address on the current device (looked up once per device; returns a
// hipError_t, 0 on success).
size_t static_scratch_bytes();
int static_scratch(void** ptr);

// Scratch bytes the plan chosen for `a` needs (0: no split-K).  Split-K is
// only planned when a.ws is non-null.
size_t conv_pw_ws_bytes(const ConvArgs& a);
size_t conv_patch_ws_bytes(const ConvArgs& a);

// Plan of the few-input-channel kernel (C <= 4, e.g. an RGB stem).
struct SmallcPlan {
  int FP;     // 32-pixel tiles per wave (block: 64 channels x 128*FP pixel slots)
  int NH;     // k-steps per kernel row (taps padded to 4*NH)
  int P;      // input positions per staging load (1 or 8)
  int TR;     // output rows per block
  int PR;     // patch rows
  int PWc;    // patch columns (cells), even
  int nrb;    // row blocks per image
  int nmb;    // output-channel blocks
  int lds;    // bytes of LDS
  int w_vec;  // weights 16-byte aligned: staged with vector loads
};

// Launchers (return a hipError_t as int).  `stream` is a hipStream_t.
// One translation unit per input type keeps the builds parallel.
int launch_gemm_f32(const GemmArgs& a, int tile, void* stream);
int launch_gemm_bf16(const GemmArgs& a, int tile, void* stream);
int launch_gemm_i8(const GemmArgs& a, int tile, void* stream);
// split-K float Gemm (32x64 tiles): S slices of kslice along K, fp32
// partials in ws [S][rows][cols], then the reduction with the epilogue
int launch_gemm_splitk_f32(const GemmArgs& a, int S, int kslice, float* ws, void* stream);
int launch_gemm_splitk_bf16(const GemmArgs& a, int S, int kslice, float* ws, void* stream);
// kind: 0 = implicit GEMM (any kernel / stride / pad / dilation / group),
//       1 = 1x1 stride-1 unpadded convolution (a per-image GEMM on NCHW).
int launch_conv_f32(const ConvArgs& a, int kind, int tile, void* stream);
int launch_conv_bf16(const ConvArgs& a, int kind, int tile, void* stream);
int launch_conv_i8(const ConvArgs& a, int kind, int tile, void* stream);
// depthwise (group == C == M), VALU only
int launch_conv_depthwise(const ConvArgs& a, void* stream);
// whether the depthwise kernel's LDS band fits this geometry (host only)
bool depthwise_fits(const ConvArgs& a);
// depthwise 3x3 with one row segment per lane (pads 1, stride 1 or 2, fp32 / bf16)
bool depthwise_rows_applicable(const ConvArgs& a);
int launch_conv_depthwise_rows(const ConvArgs& a, void* stream);
const char* conv_depthwise_rows_describe(const ConvArgs& a, char* buf, int cap);
// 3x3 bf16 convolution with an LDS-staged input patch (group 1, C % 32 == 0)
bool conv_patch_geometry(const ConvArgs& a);      // dtype/shape conditions only
bool conv_patch_applicable(const ConvArgs& a);
// few-input-channel kernel (bf16, C <= 4, group 1, stride 1 or 2, no dilation, kW <= 8)
bool conv_smallc_applicable(const ConvArgs& a);
int launch_conv_smallc(const ConvArgs& a, void* stream);
const char* conv_smallc_describe(const ConvArgs& a, char* buf, int cap);
// DMA-staged pointwise kernel (bf16, 1x1, stride 1, unpadded, group 1,
// C % 32 == 0, H*W even; X aligned to its DMA piece, W 16-byte aligned; a
// residual needs H*W % 8 == 0 and 16-byte aligned X, Y and R)
bool conv_pwd_applicable(const ConvArgs& a);
int launch_conv_pwd(const ConvArgs& a, void* stream);
const char* conv_pwd_describe(const ConvArgs& a, char* buf, int cap);
// pointwise kernel (bf16, 1x1, stride 1, unpadded, group 1, C % 32 == 0)
bool conv_pw_applicable(const ConvArgs& a);
int launch_conv_pw(const ConvArgs& a, void* stream);
const char* conv_pw_describe(const ConvArgs& a, char* buf, int cap);    // plus alignment and a plan that fits
int launch_conv_patch(const ConvArgs& a, void* stream);
const char* conv_patch_describe(const ConvArgs& a, char* buf, int cap);
// Gemm with a single output row (M = 1): memory-bound, no MFMA
int launch_gemv(const GemmArgs& a, void* stream);

// The memory-bound steps beside the convolutions (NCHW).
struct PoolArgs {
  int dt;                 // DT_F32 or DT_BF16
  int64_t total;          // elements of X (BatchNorm)
  int64_t planes;         // N * C
  int C, HW;              // channels; plane length H * W (BatchNorm, GlobalAveragePool)
  int H, W, Ho, Wo, kH, kW, sh, sw, pt, pl, dh, dw;   // MaxPool window geometry
  const void* X;
  void* Y;
  const float* gamma;     // BatchNorm parameters, fp32, [C]
  const float* beta;
  const float* mean;
  const float* var;
  float eps;
  int act;
};
int launch_bn_act(const PoolArgs& a, void* stream);
// MaxPool on the depthwise kernel's staged band (group == C == M, f32 / bf16)
// Weight-only int4 MatMul (MatMulNBits, 4 bits, blocks of 32 along K).
struct NBitsArgs {
  int M, N, K, nblk;      // nblk = ceil(K / 32)
  const void* A;          // bf16 [M, K], row stride lda
  int64_t lda;
  bool a_vec;             // A 16-byte aligned with lda % 8 == 0
  const uint8_t* B;       // [N][nblk][16] packed nibbles
  const float* scales;    // [N][nblk]
  const uint8_t* zp;      // [N][(nblk + 1) / 2] packed nibbles, or null (8)
  const void* bias;       // bf16 [N] or null
  void* Y;                // bf16 [M, N], row stride ldy
  int64_t ldy;
};
int launch_matmul_nbits(const NBitsArgs& a, void* stream);

size_t dynq_workspace_bytes();
int launch_dynamic_quantize(int64_t n, const float* X, uint8_t* Y, float* y_scale, uint8_t* y_zp,
                            void* ws, void* stream);
int launch_maxpool_dw(const ConvArgs& a, void* stream);
int launch_maxpool(const PoolArgs& a, void* stream);
int launch_global_avgpool(const PoolArgs& a, void* stream);

}  // namespace ox
