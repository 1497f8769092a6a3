/*
 * oxref.h -- plain, slow, obviously-correct CPU oracle for the fused
 * GEMM / implicit-GEMM convolution path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the product
 * library (libox) and nothing else.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load or call it.  It shares no
 * source, header, table or helper with the GPU library, and the GPU library
 * never calls it: there is no CPU fallback anywhere in the product.
 *
 * What it computes (each function cites the passage it follows):
 *   - ONNX MatMul (batched) and Gemm with a fused activation, as written in
 *     the "Cuda Executor" section of the Kyanite README (matmul with
 *     transposed inputs, alpha scalars) and the "True batched MatMul/Gemm
 *     dispatch" item of "OxiONNX 0.1.7 Released".
 *   - ONNX Conv (cross-correlation, explicit pads, stride, dilation, group)
 *     by direct summation, as the convolution OxiONNX picks kernels for in its
 *     "Technical Deep Dive", item 2 (ImplicitGemmConv / Conv1x1 / DepthwiseConv
 *     all compute this one sum).
 *   - Inference BatchNorm (unfused: divide by the standard deviation), as in
 *     the Kyanite "Cuda Executor" autokernel example, and the offline
 *     BatchNorm fold W' = scale*W, bias = shift of the tensorforge
 *     "ResNet fusion" paragraph.
 *   - The activations ReLU, ReLU6 (a clamp, Kyanite "Optimizer") and GELU
 *     (the Gelu composite of the Onyxia README, read as the exact erf form).
 *   - Static int8 (QLinearConv / QLinearMatMul with int32 bias) as listed in
 *     the onnx-vulkan-rs feature list, with int64 accumulation and a fixed
 *     fp64 requantisation with round-half-to-even; and the same with uint8
 *     activations or outputs and per-channel weight zero points (the full
 *     zero-point correction of the onnx-vulkan-rs design notes).
 *
 * Floating point: every input arrives as double (fp32 and bf16 values widen
 * exactly); sums run in double in a fixed loop order (channel, then kernel
 * row, then kernel column; or k ascending).  OpenMP splits the work over
 * output elements only, so a result is bit-identical for any thread count.
 *
 * Return value of every function: 0 on success, a negative number for an
 * argument the oracle refuses (see each function).
 */
#ifndef OXREF_H
#define OXREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OXREF_ACT_NONE = 0, OXREF_ACT_RELU = 1, OXREF_ACT_RELU6 = 2, OXREF_ACT_GELU = 3 };

/* Error codes returned by the oracle. */
enum {
  OXREF_OK = 0,
  OXREF_EARG = -1,      /* null pointer, negative size, unknown enum */
  OXREF_ESHAPE = -2,    /* output size below 1, group does not divide */
  OXREF_ERANGE = -3     /* an int8 accumulator would not fit in int32 */
};

/* Convolution shape.  Pads follow the ONNX order [top, left, bottom, right]. */
typedef struct {
  int64_t N, C, H, W;      /* input NCHW */
  int64_t M, kH, kW;       /* output channels, kernel size */
  int64_t s_h, s_w;        /* strides */
  int64_t p_t, p_l, p_b, p_r;
  int64_t d_h, d_w;        /* dilations */
  int64_t group;
} oxref_conv;

/* Thread control (the determinism check runs the oracle at 1 and N threads). */
int oxref_set_threads(int n);
int oxref_get_threads(void);

/* Activation on one value and on an array, in double. */
double oxref_act1(int act, double v);
int oxref_act(int act, int64_t n, double* v);

/* ONNX MatMul, batched: C[b,i,j] = sum_k A[b,i,k] * B[b',k,j] with b' = b, or
 * b' = 0 when sB == 0 (B broadcast over the batch).  sA / sB are the batch
 * strides in elements (sA must be M*K; sB is N*K or 0).  C is [batch,M,N]. */
int oxref_matmul(int64_t batch, int64_t M, int64_t N, int64_t K,
                 const double* A, int64_t sA, const double* B, int64_t sB,
                 double* C);

/* ONNX Gemm with a fused activation:
 *   Y[i,j] = act(alpha * sum_k A'[i,k] * B'[k,j] + beta * bias[j])
 * A' = A^T when transA (A stored [K,M]), else A ([M,K]); B' = B^T when transB
 * (B stored [N,K]), else B ([K,N]).  bias is [N] or NULL (then no bias term).
 * Y is [M,N] row-major. */
int oxref_gemm(int64_t M, int64_t N, int64_t K, int transA, int transB,
               double alpha, const double* A, const double* B, double beta,
               const double* bias, int act, double* Y);
/* The same, evaluated only at the flat output indices idx[0..npts). */
int oxref_gemm_at(int64_t M, int64_t N, int64_t K, int transA, int transB,
                  double alpha, const double* A, const double* B, double beta,
                  const double* bias, int act, int64_t npts, const int64_t* idx,
                  double* out);

/* Output spatial size of an ONNX Conv; OXREF_ESHAPE when below 1. */
int oxref_conv_out_dims(const oxref_conv* d, int64_t* Ho, int64_t* Wo);

/* ONNX Conv by direct summation, plus bias and activation:
 *   Y[n,m,oh,ow] = act(b[m] + sum_{c,kh,kw} X[n, gm*C/g + c, ih, iw] * W[m,c,kh,kw])
 * ih = oh*s_h - p_t + kh*d_h, iw = ow*s_w - p_l + kw*d_w, terms outside the
 * input skipped, gm = m / (M/g).  W is [M, C/g, kH, kW]; b is [M] or NULL. */
int oxref_conv2d(const oxref_conv* d, const double* X, const double* Wt,
                 const double* b, int act, double* Y);
int oxref_conv2d_at(const oxref_conv* d, const double* X, const double* Wt,
                    const double* b, int act, int64_t npts, const int64_t* idx,
                    double* out);

/* The same with a residual input R of the output's shape [N, M, Ho, Wo] (or
 * NULL), added after the bias and before the activation:
 *   Y[o] = act((b[m] + conv sum) + R[o])
 * -- the fused "convolution + residual + bias + relu" operation that the
 * Kyanite README ("Cuda Executor", operator fusion) plans for cuDNN, with any
 * of the activations here. */
int oxref_conv2d_res(const oxref_conv* d, const double* X, const double* Wt,
                     const double* b, const double* R, int act, double* Y);
int oxref_conv2d_res_at(const oxref_conv* d, const double* X, const double* Wt,
                        const double* b, const double* R, int act, int64_t npts,
                        const int64_t* idx, double* out);

/* ONNX BatchNormalization (inference), in place on Y [N, M, HW]:
 *   z = (y - mean[m]) / sqrt(var[m] + eps) * gamma[m] + beta[m]. */
int oxref_batchnorm(int64_t N, int64_t M, int64_t HW, double* Y,
                    const double* gamma, const double* beta, const double* mean,
                    const double* var, double eps);

/* ONNX MaxPool (NCHW, ceil_mode 0): the window of ONNX Conv's geometry in
 * d (kH, kW, strides, pads, dilations; C planes, d->M and d->group unused),
 * each output the largest input under it; padding cells never win (-inf).
 * ONNX GlobalAveragePool: Y[n,c] = (1/HW) * sum over the plane, summed in
 * order.  Both are the classifier-head / stem steps next to the convolutions
 * in the ResNet pipelines of tensorforge ("ResNet fusion") and onnx-vulkan-rs
 * (the CNN operator list). */
int oxref_maxpool2d(const oxref_conv* d, const double* X, double* Y);
int oxref_global_avgpool(int64_t N, int64_t C, int64_t HW, const double* X, double* Y);

/* Offline BatchNorm fold, in double:
 *   scale = gamma / sqrt(var + eps), shift = beta - mean * scale
 *   W'[m,:] = scale[m] * W[m,:],  b'[m] = scale[m] * b0[m] + shift[m]
 * W is [M, Kper]; b0 is [M] or NULL (read as zero). */
int oxref_fold_batchnorm(int64_t M, int64_t Kper, const double* W, const double* b0,
                         const double* gamma, const double* beta,
                         const double* mean, const double* var, double eps,
                         double* W_out, double* b_out);

/* Static int8 convolution (QLinearConv with an int32 bias, symmetric
 * per-output-channel weights):
 *   acc[n,m,oh,ow] = bias_q[m] + sum over in-bounds taps (xq - x_zp) * wq
 * in int64 (OXREF_ERANGE if any |acc| >= 2^31), then
 *   mult[m] = ((double)x_s * (double)w_s[m]) / (double)y_s
 *   y = clamp(rint((double)acc * mult[m]) + y_zp, -128, 127)
 * with the default rounding mode (half to even).  acc_out (int64, may be NULL)
 * receives acc; y_out (may be NULL) receives y. */
int oxref_conv2d_int8(const oxref_conv* d, const int8_t* xq, const int8_t* wq,
                      const int32_t* bias_q, int32_t x_zp, float x_s,
                      const float* w_s, float y_s, int32_t y_zp,
                      int64_t* acc_out, int8_t* y_out);

/* Static int8 Gemm (QLinearMatMul with bias, weights stored [N,K]):
 *   acc[i,j] = bias_q[j] + sum_k (xq[i,k] - x_zp) * wq[j,k]
 * then the same requantisation with the channel index j. */
int oxref_gemm_int8(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                    const int8_t* wq, const int32_t* bias_q, int32_t x_zp,
                    float x_s, const float* w_s, float y_s, int32_t y_zp,
                    int64_t* acc_out, int8_t* y_out);

/* Quantised convolution with both zero points (QLinearConv / ConvInteger as
 * the onnx-vulkan-rs design notes write the zero-point correction: every
 * product is (x - x_zp) * (w - w_zp)).  Activations and weights arrive as
 * int32 holding their stored integers (int8 or uint8 values); the weight
 * zero point is per output channel (w_zp [M], NULL = all 0):
 *   acc[n,m,oh,ow] = bias_q[m] + sum over in-bounds taps (x - x_zp) * (w - w_zp[m])
 * (a tap in the padding holds the value x_zp and contributes nothing), in
 * int64 (OXREF_ERANGE if any |acc| >= 2^31), then
 *   y = clamp(rint((double)acc * mult[m]) + y_zp, y_lo, y_hi)
 * with mult[m] as above and [y_lo, y_hi] = [-128, 127] (int8 output) or
 * [0, 255] (uint8 output).  acc_out / y_out may be NULL. */
int oxref_qconv2d(const oxref_conv* d, const int32_t* x, const int32_t* w,
                  const int32_t* bias_q, int32_t x_zp, const int32_t* w_zp, float x_s,
                  const float* w_s, float y_s, int32_t y_zp, int32_t y_lo, int32_t y_hi,
                  int64_t* acc_out, int32_t* y_out);

/* The same for a Gemm / MatMulInteger, X [M,K], W stored [N,K], channel j:
 *   acc[i,j] = bias_q[j] + sum_k (x[i,k] - x_zp) * (w[j,k] - w_zp[j]) */
int oxref_qgemm(int64_t M, int64_t N, int64_t K, const int32_t* x, const int32_t* w,
                const int32_t* bias_q, int32_t x_zp, const int32_t* w_zp, float x_s,
                const float* w_s, float y_s, int32_t y_zp, int32_t y_lo, int32_t y_hi,
                int64_t* acc_out, int32_t* y_out);

/* The requantisation step alone, for one accumulator (used by the tie and
 * saturation checks). */
int32_t oxref_requant1(int64_t acc, float x_s, float w_s, float y_s, int32_t y_zp);

#ifdef __cplusplus
}
#endif
#endif
