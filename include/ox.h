/*
 * ox.h -- C ABI of libox, a fused GEMM / implicit-GEMM convolution library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes the path that ONNX runtimes share for their heaviest
 * operators: ONNX MatMul (batched) and Gemm, and ONNX Conv lowered to an
 * implicit GEMM, each with a fused epilogue -- a bias (usually a BatchNorm
 * folded offline into the weights), then ReLU, ReLU6 or GELU -- and a static
 * int8 path with int32 accumulation and round-half-to-even requantisation.
 *
 * Conventions shared by every call below:
 *   - Tensors are dense, row-major (ONNX / NCHW).  Element sizes: fp32 4 B,
 *     bf16 2 B (raw bfloat16 bits), int8 1 B, int32 4 B.
 *   - Pointers named as DEVICE pointers are caller-owned device memory that
 *     must stay valid until the work enqueued on `stream` completes.  The
 *     library keeps no reference after returning, allocates no memory,
 *     creates no streams or events and holds no global mutable state beyond a
 *     per-thread error message.  Calls are re-entrant.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Hot-path calls are asynchronous: they validate every argument
 *     on the host, enqueue kernels on `stream` and return.  Nothing is
 *     enqueued when validation fails.
 *   - Any pointer alignment is accepted: kernels pick the widest vector
 *     access the pointers and strides permit.
 *   - Every tensor must hold fewer than 2^31 elements (OX_ERR_UNSUPPORTED
 *     otherwise).  Empty tensors (a zero dimension) are accepted and enqueue
 *     nothing (except a Gemm with K = 0, which still writes act(beta*bias)).
 *   - Errors: a non-zero ox_status; ox_last_error() then names the offending
 *     argument.  A failing HIP launch returns OX_ERR_HIP; device faults
 *     surface at the caller's next synchronisation.  There is no fallback:
 *     an unsupported combination is refused, never approximated.
 *   - OX_FORCE_KERNEL=<variant> in the environment forces a kernel variant
 *     where it is applicable (for A/B measurements); OX_LOG=1 prints the
 *     selected variant of each call to stderr.
 */
#ifndef OX_H
#define OX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OX_OK = 0,
  OX_ERR_INVALID_ARG = 1,   /* null pointer, negative size, unknown enum */
  OX_ERR_SHAPE = 2,         /* shapes that do not fit together (e.g. output size < 1) */
  OX_ERR_UNSUPPORTED = 3,   /* valid ONNX, but not a combination this library runs */
  OX_ERR_HIP = 4            /* a HIP runtime call failed */
} ox_status;

typedef enum { OX_F32 = 0, OX_BF16 = 1, OX_I8 = 2, OX_I32 = 3 } ox_dtype;

/* Fused activations.  ReLU = max(v,0); ReLU6 = min(max(v,0),6) (the clamp the
 * Kyanite README "Optimizer" section merges relu/min/max into); GELU is the
 * exact erf form 0.5*v*(1+erf(v/sqrt(2))) (the Gelu composite of the Onyxia
 * README). */
typedef enum { OX_ACT_NONE = 0, OX_ACT_RELU = 1, OX_ACT_RELU6 = 2, OX_ACT_GELU = 3 } ox_act;

/* ONNX Conv geometry.  Input X [N, C, H, W], weights [M, C/group, kH, kW],
 * output Y [N, M, Ho, Wo] with
 *   Ho = floor((H + p_t + p_b - d_h*(kH-1) - 1) / s_h) + 1   (Wo likewise).
 * Pads are explicit, in the ONNX order [top, left, bottom, right], and may be
 * asymmetric; auto_pad is the caller's to resolve. */
typedef struct {
  int64_t N, C, H, W;
  int64_t M, kH, kW;
  int64_t s_h, s_w;
  int64_t p_t, p_l, p_b, p_r;
  int64_t d_h, d_w;
  int64_t group;
} ox_conv_desc;

/* ---------------------------------------------------------------- hot path */

/* ONNX MatMul, batched ("True batched MatMul/Gemm dispatch" of "OxiONNX 0.1.7
 * Released": one launch for the whole batch, not one per batch element).
 *   C[b,i,j] = sum_k A[b,i,k] * B[b',k,j],  b' = b, or 0 when sB == 0.
 * t: OX_F32 or OX_BF16 (A, B and C all of type t; fp32 accumulation).
 * A: DEVICE [batch, M, K], batch stride sA elements (sA >= M*K; A rows dense).
 * B: DEVICE [batch, K, N], batch stride sB = 0 (broadcast) or >= K*N.
 * C: DEVICE [batch, M, N], dense, written in full. */
ox_status ox_matmul_batched(ox_dtype t, int64_t batch, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t sA, const void* B, int64_t sB,
                            void* C, void* stream);

/* ONNX Gemm with a fused activation (the GEMM-epilogue fusion of the
 * tensorforge "Status" table and "ResNet fusion" paragraph; transposed
 * inputs and scalar operands as in the Kyanite "Cuda Executor" section):
 *   Y[i,j] = act(alpha * sum_k A'[i,k] * B'[k,j] + beta * bias[j])
 * A' = A^T when transA (A stored [K,M]) else A ([M,K]);
 * B' = B^T when transB (B stored [N,K]) else B ([K,N]).
 * t = OX_F32 / OX_BF16: A, B, bias and Y of type t, fp32 accumulation; bias
 *   is DEVICE [N] or NULL; int8_params must be NULL.
 * t = OX_I8 / OX_I32: static int8 (QLinearMatMul with an int32 bias):
 *   A = x_q DEVICE int8 [M,K] (transA = 0), B = w_q DEVICE int8 [N,K]
 *   (transB = 1), int8_params = DEVICE block made by ox_int8_prepare for N
 *   channels, bias = NULL, alpha = beta = 1, act = OX_ACT_NONE.
 *   OX_I8 writes requantised int8 Y [M,N]; OX_I32 writes the int32
 *   accumulators acc[i,j] = bias_q[j] + sum_k (x_q[i,k] - x_zp) * w_q[j,k]. */
ox_status ox_gemm_fused(ox_dtype t, int64_t M, int64_t N, int64_t K, int transA, int transB,
                        float alpha, const void* A, const void* B, float beta,
                        const void* bias, ox_act act, void* Y, const void* int8_params,
                        void* stream);

/* The same float Gemm (t = OX_F32 / OX_BF16) with a caller-owned workspace
 * that lets a problem too small to fill the GPU split its reduction: K is
 * cut into slices whose fp32 partial products go to the workspace
 * ([slices][M][N]) and a second kernel adds them in slice order before
 * alpha, beta * bias and the activation (so the sum order differs from
 * ox_gemm_fused's; the tolerance of a float Gemm covers it).  workspace:
 * DEVICE, 16-byte aligned, at least ox_gemm_workspace_bytes(t, M, N, K)
 * bytes (0 = no split planned: the call is then ox_gemm_fused; workspace
 * may be NULL); calls sharing a workspace must not overlap. */
size_t ox_gemm_workspace_bytes(ox_dtype t, int64_t M, int64_t N, int64_t K);
ox_status ox_gemm_fused_ws(ox_dtype t, int64_t M, int64_t N, int64_t K, int transA, int transB,
                           float alpha, const void* A, const void* B, float beta,
                           const void* bias, ox_act act, void* Y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ONNX Conv + bias + activation, float path (Conv -> BatchNorm -> Relu folded
 * into one fused convolution, tensorforge "ResNet fusion"; per-shape choice
 * of an implicit-GEMM, a 1x1 and a depthwise kernel, "OxiONNX 0.1.7
 * Released", Technical Deep Dive item 2):
 *   Y[n,m,oh,ow] = act(bias[m] + sum_{c,kh,kw} X[n, g*C/group + c, ih, iw] * W[m,c,kh,kw])
 *   ih = oh*s_h - p_t + kh*d_h, iw = ow*s_w - p_l + kw*d_w (zero outside),
 *   g = m / (M/group).
 * t: OX_F32 or OX_BF16 (X, W, bias, Y all of type t; fp32 accumulation).
 * X: DEVICE [N,C,H,W]; W: DEVICE [M, C/group, kH, kW] (ONNX layout, e.g. the
 * output of ox_fold_batchnorm); bias: DEVICE [M] or NULL; Y: DEVICE
 * [N,M,Ho,Wo], written in full.  No im2col buffer is ever materialised. */
ox_status ox_conv2d_fused(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                          const void* bias, ox_act act, void* Y, void* stream);

/* Static int8 ONNX Conv (QLinearConv with an int32 bias, symmetric
 * per-output-channel weights, per-tensor activation scale and zero point;
 * onnx-vulkan-rs feature list, "Static int8 (QOperator)"):
 *   acc[n,m,oh,ow] = bias_q[m] + sum over in-bounds taps (x_q - x_zp) * w_q
 *   y = clamp(rint(acc * mult[m]) + y_zp, -128, 127),
 *   mult[m] = ((double)x_s * (double)w_s[m]) / (double)y_s, rint half-to-even.
 * Xq: DEVICE int8 [N,C,H,W]; Wq: DEVICE int8 [M, C/group, kH, kW];
 * int8_params: DEVICE block from ox_int8_prepare for these weights;
 * y_type: OX_I8 (requantised int8 Y) or OX_I32 (the int32 accumulators);
 * Y: DEVICE [N,M,Ho,Wo]. */
ox_status ox_conv2d_int8(const ox_conv_desc* d, const int8_t* Xq, const int8_t* Wq,
                         const void* int8_params, ox_dtype y_type, void* Y, void* stream);

/* The kernel variant ox_conv2d_fused (t = OX_F32 / OX_BF16) or ox_conv2d_int8
 * (t = OX_I8) would launch for this geometry, as "<kind>/<dtype>[/<tile>]"
 * with kind dw, 1x1 or igemm (e.g. "igemm/bf16/64x128"), honouring
 * OX_FORCE_KERNEL.  Host only, enqueues nothing; the shape choice follows the
 * per-shape selection of "OxiONNX 0.1.7 Released" (Technical Deep Dive, item
 * 2).  name: HOST buffer of cap bytes (NUL-terminated, truncated to fit). */
ox_status ox_conv2d_variant(ox_dtype t, const ox_conv_desc* d, char* name, size_t cap);

/* Convolution with weights packed offline by ox_conv2d_pack_weights.  Same
 * operation, arguments and errors as ox_conv2d_fused; Wp is the DEVICE copy
 * of the packed weights.  Only geometries for which
 * ox_conv2d_packed_weights_bytes() is non-zero have a packed form; those run
 * the LDS-patch implicit-GEMM kernel, and OX_ERR_UNSUPPORTED is returned when
 * X or Wp is not 16-byte aligned. */
ox_status ox_conv2d_fused_packed(ox_dtype t, const ox_conv_desc* d, const void* X, const void* Wp,
                                 const void* bias, ox_act act, void* Y, void* stream);

/* Scratch bytes that ox_conv2d_fused_ws may use for this geometry: the fp32
 * partial tiles of a channel-split (split-K) plan, which the 1x1 and the
 * LDS-patch 3x3 kernels choose when a layer has too few output tiles to
 * occupy the chip (the deep, small-spatial layers of an image network).
 * 0 when no split is planned.  Host only; honours OX_FORCE_KERNEL. */
size_t ox_conv2d_workspace_bytes(ox_dtype t, const ox_conv_desc* d);

/* ox_conv2d_fused (w_packed = 0, W in ONNX layout) or ox_conv2d_fused_packed
 * (w_packed = 1, W packed by ox_conv2d_pack_weights) with a caller-owned
 * scratch buffer, so that the kernels may split a tile's channel range into
 * slices that write fp32 partials and a second pass adds them in slice order
 * (the result does not depend on timing).  The library allocates nothing.
 * workspace: DEVICE, 16-byte aligned, at least
 * ox_conv2d_workspace_bytes(t, d) bytes (workspace_bytes says how many), or
 * NULL for no split (then identical to the calls above).  Its contents on
 * entry do not matter and are garbage afterwards; calls that share it must
 * be ordered on one stream.  Errors as ox_conv2d_fused, plus
 * OX_ERR_INVALID_ARG for a misaligned or too small workspace. */
ox_status ox_conv2d_fused_ws(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                             int w_packed, const void* bias, ox_act act, void* Y, void* workspace,
                             size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ox_conv2d_fused_ws with the scratch taken from a device array inside the
 * library instead of a caller workspace.  Same operation, arguments (minus
 * the workspace) and errors as ox_conv2d_fused_ws; no hipMalloc, hipFree or
 * other allocation, here or in the kernels.
 * The array holds ox_static_scratch_bytes() bytes (32 MiB) on every GPU the
 * library runs on, for the life of the process; its address on a device is
 * looked up on the first call made with that device current.  A geometry
 * whose split-K plan needs more scratch than that is refused with
 * OX_ERR_UNSUPPORTED before anything is enqueued (ox_conv2d_workspace_bytes
 * gives the need).  All calls on one GPU share its array, which keeps the last
 * call's partials: calls that overlap on one GPU (several streams or host
 * threads) race on it and must be ordered by the caller. */
size_t ox_static_scratch_bytes(void);
ox_status ox_conv2d_fused_static(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                                 int w_packed, const void* bias, ox_act act, void* Y, void* stream);

/* Conv + bias + residual + activation, fused:
 *   Y[n,m,oh,ow] = act((conv(X, W)[n,m,oh,ow] + bias[m]) + R[n,m,oh,ow])
 * the single "convolution + residual + bias + relu" operation that the
 * Kyanite README (section "Cuda Executor", operator fusion) plans for a
 * residual block, here with any activation: an ONNX Conv whose output feeds
 * an Add with a tensor of its own shape, then the activation.  With BatchNorm
 * folded into W and bias this is the end of a ResNet bottleneck (conv, BN,
 * + shortcut, ReLU) or of a MobileNetV2 stride-1 block (act = OX_ACT_NONE).
 * t: OX_F32 or OX_BF16; X, W (ONNX layout), bias, R and Y all of type t.
 * R: DEVICE, dense [N, M, Ho, Wo] like Y, aligned to its element size; it may
 * be Y itself (the residual is then replaced by the result); any other
 * overlap of R or Y with the inputs is undefined.  R = NULL is
 * ox_conv2d_fused_ws.  The 1x1 convolutions run on the pointwise kernel, all
 * other geometries on the implicit-GEMM tile engine (the LDS-patch,
 * depthwise and few-channel kernels take no residual).  workspace: as for
 * ox_conv2d_fused_ws (ox_conv2d_workspace_bytes(t, d) bytes suffice).
 * Errors as ox_conv2d_fused_ws, plus OX_ERR_INVALID_ARG for a misaligned R
 * and OX_ERR_UNSUPPORTED when OX_FORCE_KERNEL names a kernel without a
 * residual epilogue. */
ox_status ox_conv2d_fused_res(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                              const void* bias, const void* R, ox_act act, void* Y, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---------------------------------- memory-bound steps beside the convs */

/* ONNX BatchNormalization (inference) + activation, for a BatchNorm that
 * cannot be folded into a convolution (the pre-activation BN -> ReLU of a
 * ResNet-v2 block; tensorforge's "ResNet fusion" folds only the BN that
 * follows a conv):
 *   Y[n,c,i] = act((X[n,c,i] - mean[c]) * gamma[c] / sqrt(var[c] + eps) + beta[c])
 * computed in fp32 (the scale and shift per channel, then one multiply-add
 * per element).  X, Y: DEVICE, dense NCHW [N, C, HW] of type t (OX_F32 or
 * OX_BF16), may be the same buffer (in place).  gamma, beta, mean, var:
 * DEVICE fp32 [C].  eps > 0.  One kernel, no allocation.  Errors:
 * OX_ERR_UNSUPPORTED for another t, OX_ERR_SHAPE for negative sizes,
 * OX_ERR_INVALID_ARG for NULL or misaligned pointers, a bad act or eps. */
ox_status ox_batchnorm_act(ox_dtype t, int64_t N, int64_t C, int64_t HW, const void* X,
                           const float* gamma, const float* beta, const float* mean, const float* var,
                           float eps, ox_act act, void* Y, void* stream);

/* ONNX MaxPool (NCHW, ceil_mode 0, storage_order 0): the window geometry is
 * an ox_conv_desc with M == C and group == 1 (kH, kW, strides, pads
 * [t,l,b,r], dilations; output size as for Conv); each output is the largest
 * input under its window, padding cells never taken.  X [N, C, H, W], Y
 * [N, C, Ho, Wo], DEVICE, type t (OX_F32 or OX_BF16; bf16 maxima are exact).
 * Errors as ox_conv2d_fused, plus OX_ERR_INVALID_ARG when a pad reaches the
 * kernel extent (a window of padding only). */
ox_status ox_maxpool2d(ox_dtype t, const ox_conv_desc* d, const void* X, void* Y, void* stream);

/* ONNX GlobalAveragePool: Y[n,c] = (1/HW) * sum_i X[n,c,i], summed in fp32
 * in a fixed order (the same bits every run) and rounded to t once.
 * X [N, C, HW], Y [N, C] (i.e. [N, C, 1, 1]), DEVICE, type t (OX_F32 or
 * OX_BF16).  HW >= 1.  Errors: OX_ERR_SHAPE for HW < 1 or negative sizes,
 * OX_ERR_INVALID_ARG for NULL or misaligned pointers. */
ox_status ox_global_avgpool(ox_dtype t, int64_t N, int64_t C, int64_t HW, const void* X, void* Y,
                            void* stream);

/* ------------------------------------------------- offline, host, untimed */

/* Size in bytes of the packed weights of a convolution, or 0 when this
 * geometry has no packed form (today: bf16, 3x3, group 1, C % 32 == 0,
 * equal strides of 1 or 2).  The packed size equals the ONNX size. */
size_t ox_conv2d_packed_weights_bytes(ox_dtype t, const ox_conv_desc* d);

/* Offline weight preparation (the weight half of the "weight/params prep"
 * step that the BatchNorm fold begins): reorder ONNX weights W[M][C][kH][kW]
 * into blocks of 32 input channels, tap-major,
 *   Wp[m][c/32][kh*kW + kw][c%32] = W[m][c][kh][kw],
 * so that the kernel copies each block's operand tile into LDS as it lies.
 * W_host, Wp_host: HOST buffers of ox_conv2d_packed_weights_bytes(t, d) bytes. */
ox_status ox_conv2d_pack_weights(ox_dtype t, const ox_conv_desc* d, const void* W_host, void* Wp_host);

/* BatchNorm fold (tensorforge "ResNet fusion": W' = scale*W, bias = shift;
 * Kyanite "Optimizer": consecutive affine ops merged into one scale + bias,
 * division by a constant replaced by a multiplication).  Host memory, fp64
 * arithmetic, fp32 results:
 *   scale[m] = gamma[m] / sqrt(var[m] + eps);  shift[m] = beta[m] - mean[m]*scale[m]
 *   W_out[m,k] = scale[m]*W[m,k];  b_out[m] = scale[m]*b0[m] + shift[m]
 * W, W_out: HOST [M, Kper]; b0: HOST [M] or NULL (zero); gamma, beta, mean,
 * var, b_out: HOST [M].  W_out may alias W. */
ox_status ox_fold_batchnorm(int64_t M, int64_t Kper, const float* W, const float* b0,
                            const float* gamma, const float* beta, const float* mean,
                            const float* var, float eps, float* W_out, float* b_out);

/* Size in bytes of the int8 parameter block for M output channels
 * (a 32-byte header, then 8 B fp64 multiplier + 4 B folded int32 bias + 4 B
 * weight zero point per channel). */
size_t ox_int8_params_bytes(int64_t M);

/* Prepare the int8 parameter block on the host, once per layer.  Host fp64:
 *   mult[m]      = ((double)x_scale * (double)w_scale[m]) / (double)y_scale
 *   bias_fold[m] = bias_q[m] - x_zp * sum_k Wq[m,k]
 * The fold is the zero-point correction of the onnx-vulkan-rs design notes
 * with a weight zero point of 0; the kernels therefore pad with x_zp.
 * Wq_host: HOST int8 [M, Kper]; w_scale: HOST [M] (> 0); bias_q: HOST [M] or
 * NULL; x_zp, y_zp in [-128, 127]; scales finite and > 0.
 * params_host_out: HOST, ox_int8_params_bytes(M) bytes; the caller copies it
 * to the device and passes that copy to the int8 calls.
 * Range: the accumulators are int32.  A channel m is refused
 * (OX_ERR_UNSUPPORTED, naming m) when some input could take it outside
 * int32: bias_q[m] + sum_k (x - x_zp) * w[m,k] over every x the activation
 * type allows, or the kernels' raw sum_k x * w[m,k] before the folded bias.
 * The bound is exact per channel (computed from the weights), so e.g.
 * Kper = 65793 weights of -128 with x_zp = -128 pass and 65794 do not. */
ox_status ox_int8_prepare(int64_t M, int64_t Kper, const int8_t* Wq_host, const float* w_scale,
                          float x_scale, int32_t x_zp, float y_scale, int32_t y_zp,
                          const int32_t* bias_q, void* params_host_out);

/* The parameter block for the other quantisation variants (QLinearConv /
 * QLinearMatMul with uint8 activations or outputs and per-channel weight
 * zero points; ConvInteger / MatMulInteger through OX_I32 outputs), with
 * the full zero-point correction of the onnx-vulkan-rs design notes:
 *   acc = bias_q[m] + sum over in-bounds taps (x - x_zp) * (w - w_zp[m])
 *   y   = clamp(rint(acc * mult[m]) + y_zp, lo, hi)
 * with [lo, hi] = [0, 255] when y_unsigned, else [-128, 127].  The padding
 * of a convolution holds x_zp (the quantised real zero).
 * x_unsigned: the activations given to the int8 calls are uint8 and
 * x_zp is in [0, 255] (else int8, x_zp in [-128, 127]); y_unsigned: the
 * requantised outputs are written as uint8 and y_zp is in [0, 255].
 * Wq_host: HOST int8 [M, Kper] (uint8 weights: pass w - 128 with
 * w_zp - 128, which leaves every product unchanged); w_zp: HOST int32 [M] in
 * [-128, 127] or NULL (all 0).
 * The block records the signedness: the same int8 calls (ox_gemm_fused with
 * OX_I8 / OX_I32, ox_conv2d_int8) then read and write uint8 tensors through
 * their int8_t pointers.  ox_int8_prepare(...) is this call with w_zp = NULL
 * and both flags 0. */
ox_status ox_int8_prepare_ex(int64_t M, int64_t Kper, const int8_t* Wq_host, const int32_t* w_zp,
                             const float* w_scale, float x_scale, int32_t x_zp, int x_unsigned,
                             float y_scale, int32_t y_zp, int y_unsigned, const int32_t* bias_q,
                             void* params_host_out);

/* Weight-only int4 MatMul (ONNX MatMulNBits with 4-bit weights in blocks of
 * 32 along K; the Onyxia README runs 4-bit LLM weights that stay packed on
 * the device, its prefill matmul dequantising each weight tile into shared
 * memory on load):
 *   Y[m,n] = sum_k A[m,k] * w[n,k] (+ bias[n]),
 *   w[n,k] = (q[n,k] - zp[n,k/32]) * scales[n,k/32]
 * t = OX_BF16: A [M,K], bias [N] (or NULL) and Y [M,N] bf16, row-major and
 * dense; fp32 accumulation.  Up to 4 rows (decode) run a fused
 * matrix-vector kernel that keeps the dequantised weights in fp32; more rows
 * run the MFMA tile engine, which rounds each dequantised weight to bf16.
 * A 16-byte aligned B is needed for the decode kernel (else the tile engine
 * runs those rows too).
 * B: DEVICE uint8 [N][ceil(K/32)][16]: element k of block b of row n in byte
 * (k%32)/2 of that block, the low nibble for even k (4-byte aligned).
 * scales: DEVICE fp32 [N][ceil(K/32)].  zero_points: DEVICE uint8
 * [N][ceil(ceil(K/32)/2)], block b's zero point in byte b/2, the low nibble
 * for even b; NULL means 8 for every block.  bits must be 4 and block_size
 * 32 (OX_ERR_UNSUPPORTED otherwise). */
ox_status ox_matmul_nbits(ox_dtype t, int64_t M, int64_t N, int64_t K, int bits, int block_size,
                          const void* A, const uint8_t* B, const float* scales,
                          const uint8_t* zero_points, const void* bias, void* Y, void* stream);

/* Dynamic per-tensor quantisation of fp32 activations to uint8 (ONNX
 * DynamicQuantizeLinear; the onnx-vulkan-rs notes name dynamically
 * quantised graphs, whose scale follows the tensor's extremes):
 *   lo = min(0, min X), hi = max(0, max X), y_scale = (hi - lo) / 255,
 *   y_zp = rint(clamp(-lo / y_scale, 0, 255)),
 *   Y = clamp(rint(X / y_scale) + y_zp, 0, 255)
 * in fp32 (correctly rounded division, round half to even).  An all-zero X
 * (or n = 0) gives y_scale = 0, y_zp = 0, Y = 0.  NaN inputs are not
 * supported (min / max skip them; their Y is 0).
 * X: DEVICE fp32 [n] (4-byte aligned; 16-byte aligned X with 4-byte aligned
 * Y takes the vector path); Y: DEVICE uint8 [n]; y_scale: DEVICE fp32 [1];
 * y_zp: DEVICE uint8 [1]; workspace: DEVICE, 16-byte aligned, at least
 * ox_dynamic_quantize_workspace_bytes() bytes, owned by the caller (two
 * launches on `stream`; calls that share a workspace must not overlap).
 * y_scale / y_zp then feed ox_int8_prepare_ex-style consumers (x_unsigned). */
size_t ox_dynamic_quantize_workspace_bytes(void);
ox_status ox_dynamic_quantize_linear(int64_t n, const float* X, uint8_t* Y, float* y_scale,
                                     uint8_t* y_zp, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* The message of the last failing call on this thread ("" if none). */
const char* ox_last_error(void);

/* Library version string. */
const char* ox_version(void);

#ifdef __cplusplus
}
#endif
#endif
