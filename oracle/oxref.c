/*
 * oxref.c -- the CPU oracle (test infrastructure only; see oxref.h).
 *
 * Plain loops, fp64 sums in a fixed order, direct convolution.  No BLAS, no
 * SIMD intrinsics, no im2col, no blocking.  Built with gcc
 * -O2 -fopenmp -ffp-contract=off so that no multiply-add is fused behind the
 * reader's back.
 */
#include "oxref.h"

#include <math.h>
#include <stddef.h>
#include <omp.h>

int oxref_set_threads(int n) {
  int prev = omp_get_max_threads();
  if (n > 0) omp_set_num_threads(n);
  return prev;
}

int oxref_get_threads(void) { return omp_get_max_threads(); }

/* ReLU = max(v, 0); ReLU6 = min(max(v, 0), 6) (a clamp, as the Kyanite
 * "Optimizer" section merges relu/min/max into one clamp); GELU in its exact
 * form 0.5*v*(1 + erf(v/sqrt(2))), the reading taken for the Gelu composite the
 * Onyxia README lists. */
double oxref_act1(int act, double v) {
  switch (act) {
    case OXREF_ACT_RELU: return v > 0.0 ? v : 0.0;
    case OXREF_ACT_RELU6: {
      double r = v > 0.0 ? v : 0.0;
      return r < 6.0 ? r : 6.0;
    }
    case OXREF_ACT_GELU: return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
    default: return v;
  }
}

static int act_ok(int act) { return act >= OXREF_ACT_NONE && act <= OXREF_ACT_GELU; }

int oxref_act(int act, int64_t n, double* v) {
  if (!act_ok(act) || n < 0 || (n > 0 && !v)) return OXREF_EARG;
  for (int64_t i = 0; i < n; ++i) v[i] = oxref_act1(act, v[i]);
  return OXREF_OK;
}

/* ---------------------------------------------------------------- MatMul -- */

int oxref_matmul(int64_t batch, int64_t M, int64_t N, int64_t K,
                 const double* A, int64_t sA, const double* B, int64_t sB,
                 double* C) {
  if (batch < 0 || M < 0 || N < 0 || K < 0) return OXREF_EARG;
  if (batch * M * N == 0) return OXREF_OK;
  if (!A || !B || !C) return OXREF_EARG;
  if (sA != M * K) return OXREF_EARG;
  if (sB != 0 && sB != K * N) return OXREF_EARG;
  int64_t total = batch * M * N;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < total; ++o) {
    int64_t b = o / (M * N);
    int64_t i = (o / N) % M;
    int64_t j = o % N;
    const double* a = A + b * sA + i * K;
    const double* bb = B + b * sB;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += a[k] * bb[k * N + j];
    C[o] = acc;
  }
  return OXREF_OK;
}

/* ------------------------------------------------------------------ Gemm -- */

static double gemm_one(int64_t M, int64_t N, int64_t K, int transA, int transB,
                       double alpha, const double* A, const double* B, double beta,
                       const double* bias, int act, int64_t i, int64_t j) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double a = transA ? A[k * M + i] : A[i * K + k];
    double b = transB ? B[j * K + k] : B[k * N + j];
    acc += a * b;
  }
  double v = alpha * acc;
  if (bias) v += beta * bias[j];
  return oxref_act1(act, v);
}

static int gemm_args(int64_t M, int64_t N, int64_t K, const double* A,
                     const double* B, int act) {
  if (M < 0 || N < 0 || K < 0 || !act_ok(act)) return OXREF_EARG;
  if (M * N > 0 && K > 0 && (!A || !B)) return OXREF_EARG;
  return OXREF_OK;
}

int oxref_gemm(int64_t M, int64_t N, int64_t K, int transA, int transB,
               double alpha, const double* A, const double* B, double beta,
               const double* bias, int act, double* Y) {
  int rc = gemm_args(M, N, K, A, B, act);
  if (rc) return rc;
  if (M * N == 0) return OXREF_OK;
  if (!Y) return OXREF_EARG;
  int64_t total = M * N;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < total; ++o)
    Y[o] = gemm_one(M, N, K, transA, transB, alpha, A, B, beta, bias, act, o / N, o % N);
  return OXREF_OK;
}

int oxref_gemm_at(int64_t M, int64_t N, int64_t K, int transA, int transB,
                  double alpha, const double* A, const double* B, double beta,
                  const double* bias, int act, int64_t npts, const int64_t* idx,
                  double* out) {
  int rc = gemm_args(M, N, K, A, B, act);
  if (rc) return rc;
  if (npts < 0 || (npts > 0 && (!idx || !out))) return OXREF_EARG;
  for (int64_t p = 0; p < npts; ++p)
    if (idx[p] < 0 || idx[p] >= M * N) return OXREF_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npts; ++p)
    out[p] = gemm_one(M, N, K, transA, transB, alpha, A, B, beta, bias, act,
                      idx[p] / N, idx[p] % N);
  return OXREF_OK;
}

/* ------------------------------------------------------------------ Conv -- */

/* Output size of an ONNX Conv: floor((H + pads - dilation*(k-1) - 1)/stride) + 1. */
static int64_t out_len(int64_t in, int64_t pa, int64_t pb, int64_t k, int64_t s, int64_t d) {
  int64_t span = in + pa + pb - d * (k - 1) - 1;
  if (span < 0) return 0;
  return span / s + 1;
}

static int conv_check(const oxref_conv* d) {
  if (!d) return OXREF_EARG;
  if (d->N < 0 || d->C < 1 || d->H < 1 || d->W < 1 || d->M < 1 || d->kH < 1 ||
      d->kW < 1 || d->s_h < 1 || d->s_w < 1 || d->d_h < 1 || d->d_w < 1 ||
      d->group < 1 || d->p_t < 0 || d->p_l < 0 || d->p_b < 0 || d->p_r < 0)
    return OXREF_EARG;
  if (d->C % d->group || d->M % d->group) return OXREF_ESHAPE;
  return OXREF_OK;
}

int oxref_conv_out_dims(const oxref_conv* d, int64_t* Ho, int64_t* Wo) {
  int rc = conv_check(d);
  if (rc) return rc;
  int64_t ho = out_len(d->H, d->p_t, d->p_b, d->kH, d->s_h, d->d_h);
  int64_t wo = out_len(d->W, d->p_l, d->p_r, d->kW, d->s_w, d->d_w);
  if (Ho) *Ho = ho;
  if (Wo) *Wo = wo;
  return (ho < 1 || wo < 1) ? OXREF_ESHAPE : OXREF_OK;
}

/* The pre-bias sum for one output element (n, m, oh, ow). */
static double conv_sum(const oxref_conv* d, const double* X, const double* Wt,
                       int64_t n, int64_t m, int64_t oh, int64_t ow) {
  int64_t cpg = d->C / d->group;         /* input channels per group */
  int64_t gm = m / (d->M / d->group);    /* the group output channel m is in */
  double acc = 0.0;
  for (int64_t c = 0; c < cpg; ++c) {
    const double* xplane = X + ((n * d->C) + gm * cpg + c) * d->H * d->W;
    const double* wk = Wt + ((m * cpg) + c) * d->kH * d->kW;
    for (int64_t kh = 0; kh < d->kH; ++kh) {
      int64_t ih = oh * d->s_h - d->p_t + kh * d->d_h;
      if (ih < 0 || ih >= d->H) continue;
      for (int64_t kw = 0; kw < d->kW; ++kw) {
        int64_t iw = ow * d->s_w - d->p_l + kw * d->d_w;
        if (iw < 0 || iw >= d->W) continue;
        acc += xplane[ih * d->W + iw] * wk[kh * d->kW + kw];
      }
    }
  }
  return acc;
}

static int conv_inputs(const oxref_conv* d, const double* X, const double* Wt) {
  int64_t Ho, Wo;
  int rc = oxref_conv_out_dims(d, &Ho, &Wo);
  if (rc) return rc;
  if (d->N > 0 && (!X || !Wt)) return OXREF_EARG;
  return OXREF_OK;
}

int oxref_conv2d_res(const oxref_conv* d, const double* X, const double* Wt,
                     const double* b, const double* R, int act, double* Y) {
  int rc = conv_inputs(d, X, Wt);
  if (rc) return rc;
  if (!act_ok(act)) return OXREF_EARG;
  int64_t Ho, Wo;
  oxref_conv_out_dims(d, &Ho, &Wo);
  int64_t total = d->N * d->M * Ho * Wo;
  if (total == 0) return OXREF_OK;
  if (!Y) return OXREF_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < total; ++o) {
    int64_t ow = o % Wo, oh = (o / Wo) % Ho, m = (o / (Wo * Ho)) % d->M,
            n = o / (Wo * Ho * d->M);
    double v = conv_sum(d, X, Wt, n, m, oh, ow);
    if (b) v = b[m] + v;
    if (R) v = v + R[o];
    Y[o] = oxref_act1(act, v);
  }
  return OXREF_OK;
}

int oxref_conv2d(const oxref_conv* d, const double* X, const double* Wt,
                 const double* b, int act, double* Y) {
  return oxref_conv2d_res(d, X, Wt, b, NULL, act, Y);
}

int oxref_conv2d_res_at(const oxref_conv* d, const double* X, const double* Wt,
                        const double* b, const double* R, int act, int64_t npts,
                        const int64_t* idx, double* out) {
  int rc = conv_inputs(d, X, Wt);
  if (rc) return rc;
  if (!act_ok(act) || npts < 0 || (npts > 0 && (!idx || !out))) return OXREF_EARG;
  int64_t Ho, Wo;
  oxref_conv_out_dims(d, &Ho, &Wo);
  int64_t total = d->N * d->M * Ho * Wo;
  for (int64_t p = 0; p < npts; ++p)
    if (idx[p] < 0 || idx[p] >= total) return OXREF_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npts; ++p) {
    int64_t o = idx[p];
    int64_t ow = o % Wo, oh = (o / Wo) % Ho, m = (o / (Wo * Ho)) % d->M,
            n = o / (Wo * Ho * d->M);
    double v = conv_sum(d, X, Wt, n, m, oh, ow);
    if (b) v = b[m] + v;
    if (R) v = v + R[o];
    out[p] = oxref_act1(act, v);
  }
  return OXREF_OK;
}

int oxref_conv2d_at(const oxref_conv* d, const double* X, const double* Wt,
                    const double* b, int act, int64_t npts, const int64_t* idx,
                    double* out) {
  return oxref_conv2d_res_at(d, X, Wt, b, NULL, act, npts, idx, out);
}

/* ------------------------------------------------------------- BatchNorm -- */

int oxref_batchnorm(int64_t N, int64_t M, int64_t HW, double* Y,
                    const double* gamma, const double* beta, const double* mean,
                    const double* var, double eps) {
  if (N < 0 || M < 0 || HW < 0) return OXREF_EARG;
  if (N * M * HW == 0) return OXREF_OK;
  if (!Y || !gamma || !beta || !mean || !var) return OXREF_EARG;
  int64_t total = N * M * HW;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < total; ++o) {
    int64_t m = (o / HW) % M;
    Y[o] = (Y[o] - mean[m]) / sqrt(var[m] + eps) * gamma[m] + beta[m];
  }
  return OXREF_OK;
}

/* --------------------------------------------------------------- Pooling -- */

int oxref_maxpool2d(const oxref_conv* d, const double* X, double* Y) {
  int64_t Ho, Wo;
  int rc = oxref_conv_out_dims(d, &Ho, &Wo);
  if (rc) return rc;
  if (d->N < 0 || d->C < 0) return OXREF_EARG;
  int64_t total = d->N * d->C * Ho * Wo;
  if (total == 0) return OXREF_OK;
  if (!X || !Y) return OXREF_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < total; ++o) {
    int64_t ow = o % Wo, oh = (o / Wo) % Ho, nc = o / (Wo * Ho);
    const double* plane = X + nc * d->H * d->W;
    double best = -INFINITY;            /* padding never wins: it is -inf */
    for (int64_t kh = 0; kh < d->kH; ++kh) {
      int64_t ih = oh * d->s_h - d->p_t + kh * d->d_h;
      if (ih < 0 || ih >= d->H) continue;
      for (int64_t kw = 0; kw < d->kW; ++kw) {
        int64_t iw = ow * d->s_w - d->p_l + kw * d->d_w;
        if (iw < 0 || iw >= d->W) continue;
        double v = plane[ih * d->W + iw];
        if (v > best) best = v;
      }
    }
    Y[o] = best;
  }
  return OXREF_OK;
}

int oxref_global_avgpool(int64_t N, int64_t C, int64_t HW, const double* X, double* Y) {
  if (N < 0 || C < 0 || HW < 1) return OXREF_EARG;
  if (N * C == 0) return OXREF_OK;
  if (!X || !Y) return OXREF_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t nc = 0; nc < N * C; ++nc) {
    double acc = 0.0;
    for (int64_t i = 0; i < HW; ++i) acc += X[nc * HW + i];
    Y[nc] = acc / (double)HW;
  }
  return OXREF_OK;
}

int oxref_fold_batchnorm(int64_t M, int64_t Kper, const double* W, const double* b0,
                         const double* gamma, const double* beta,
                         const double* mean, const double* var, double eps,
                         double* W_out, double* b_out) {
  if (M < 0 || Kper < 0) return OXREF_EARG;
  if (M == 0) return OXREF_OK;
  if (!gamma || !beta || !mean || !var || !b_out) return OXREF_EARG;
  if (Kper > 0 && (!W || !W_out)) return OXREF_EARG;
  for (int64_t m = 0; m < M; ++m) {
    double scale = gamma[m] / sqrt(var[m] + eps);
    double shift = beta[m] - mean[m] * scale;
    for (int64_t k = 0; k < Kper; ++k) W_out[m * Kper + k] = scale * W[m * Kper + k];
    b_out[m] = scale * (b0 ? b0[m] : 0.0) + shift;
  }
  return OXREF_OK;
}

/* ------------------------------------------------------------------ int8 -- */

/* The fixed requantisation recipe: multiplier evaluated as
 * ((double)x_s * (double)w_s) / (double)y_s, then rint (half to even under
 * the default rounding mode), then the output zero point, then saturation.
 * This is the order of ONNX QuantizeLinear: round, add the zero point, clamp. */
int32_t oxref_requant1(int64_t acc, float x_s, float w_s, float y_s, int32_t y_zp) {
  double mult = ((double)x_s * (double)w_s) / (double)y_s;
  double r = rint((double)acc * mult);
  double y = r + (double)y_zp;
  if (y > 127.0) y = 127.0;
  if (y < -128.0) y = -128.0;
  return (int32_t)y;
}

static const int64_t INT32_LIMIT = 2147483648LL; /* 2^31 */

int oxref_conv2d_int8(const oxref_conv* d, const int8_t* xq, const int8_t* wq,
                      const int32_t* bias_q, int32_t x_zp, float x_s,
                      const float* w_s, float y_s, int32_t y_zp,
                      int64_t* acc_out, int8_t* y_out) {
  int64_t Ho, Wo;
  int rc = oxref_conv_out_dims(d, &Ho, &Wo);
  if (rc) return rc;
  if (x_zp < -128 || x_zp > 127 || y_zp < -128 || y_zp > 127) return OXREF_EARG;
  int64_t total = d->N * d->M * Ho * Wo;
  if (total == 0) return OXREF_OK;
  if (!xq || !wq) return OXREF_EARG;
  if (y_out && !w_s) return OXREF_EARG;
  int64_t cpg = d->C / d->group;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t o = 0; o < total; ++o) {
    int64_t ow = o % Wo, oh = (o / Wo) % Ho, m = (o / (Wo * Ho)) % d->M,
            n = o / (Wo * Ho * d->M);
    int64_t gm = m / (d->M / d->group);
    int64_t acc = bias_q ? (int64_t)bias_q[m] : 0;
    for (int64_t c = 0; c < cpg; ++c) {
      const int8_t* xplane = xq + ((n * d->C) + gm * cpg + c) * d->H * d->W;
      const int8_t* wk = wq + ((m * cpg) + c) * d->kH * d->kW;
      for (int64_t kh = 0; kh < d->kH; ++kh) {
        int64_t ih = oh * d->s_h - d->p_t + kh * d->d_h;
        if (ih < 0 || ih >= d->H) continue;
        for (int64_t kw = 0; kw < d->kW; ++kw) {
          int64_t iw = ow * d->s_w - d->p_l + kw * d->d_w;
          if (iw < 0 || iw >= d->W) continue;
          acc += ((int64_t)xplane[ih * d->W + iw] - x_zp) * (int64_t)wk[kh * d->kW + kw];
        }
      }
    }
    if (acc >= INT32_LIMIT || acc < -INT32_LIMIT) bad = 1;
    if (acc_out) acc_out[o] = acc;
    if (y_out) y_out[o] = (int8_t)oxref_requant1(acc, x_s, w_s[m], y_s, y_zp);
  }
  return bad ? OXREF_ERANGE : OXREF_OK;
}

int oxref_gemm_int8(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                    const int8_t* wq, const int32_t* bias_q, int32_t x_zp,
                    float x_s, const float* w_s, float y_s, int32_t y_zp,
                    int64_t* acc_out, int8_t* y_out) {
  if (M < 0 || N < 0 || K < 0) return OXREF_EARG;
  if (x_zp < -128 || x_zp > 127 || y_zp < -128 || y_zp > 127) return OXREF_EARG;
  if (M * N == 0) return OXREF_OK;
  if (K > 0 && (!xq || !wq)) return OXREF_EARG;
  if (y_out && !w_s) return OXREF_EARG;
  int bad = 0;
  int64_t total = M * N;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t o = 0; o < total; ++o) {
    int64_t i = o / N, j = o % N;
    int64_t acc = bias_q ? (int64_t)bias_q[j] : 0;
    for (int64_t k = 0; k < K; ++k)
      acc += ((int64_t)xq[i * K + k] - x_zp) * (int64_t)wq[j * K + k];
    if (acc >= INT32_LIMIT || acc < -INT32_LIMIT) bad = 1;
    if (acc_out) acc_out[o] = acc;
    if (y_out) y_out[o] = (int8_t)oxref_requant1(acc, x_s, w_s[j], y_s, y_zp);
  }
  return bad ? OXREF_ERANGE : OXREF_OK;
}

/* requantisation into [lo, hi] (int8 or uint8 output) */
static int32_t requant_range(int64_t acc, float x_s, float w_s, float y_s, int32_t y_zp,
                             int32_t lo, int32_t hi) {
  double mult = ((double)x_s * (double)w_s) / (double)y_s;
  double y = rint((double)acc * mult) + (double)y_zp;
  if (y > (double)hi) y = (double)hi;
  if (y < (double)lo) y = (double)lo;
  return (int32_t)y;
}

static int q_range_ok(int32_t y_zp, int32_t y_lo, int32_t y_hi) {
  if (!((y_lo == -128 && y_hi == 127) || (y_lo == 0 && y_hi == 255))) return 0;
  return y_zp >= y_lo && y_zp <= y_hi;
}

int oxref_qconv2d(const oxref_conv* d, const int32_t* x, const int32_t* w,
                  const int32_t* bias_q, int32_t x_zp, const int32_t* w_zp, float x_s,
                  const float* w_s, float y_s, int32_t y_zp, int32_t y_lo, int32_t y_hi,
                  int64_t* acc_out, int32_t* y_out) {
  int64_t Ho, Wo;
  int rc = oxref_conv_out_dims(d, &Ho, &Wo);
  if (rc) return rc;
  if (!q_range_ok(y_zp, y_lo, y_hi)) return OXREF_EARG;
  int64_t total = d->N * d->M * Ho * Wo;
  if (total == 0) return OXREF_OK;
  if (!x || !w) return OXREF_EARG;
  if (y_out && !w_s) return OXREF_EARG;
  int64_t cpg = d->C / d->group;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t o = 0; o < total; ++o) {
    int64_t ow = o % Wo, oh = (o / Wo) % Ho, m = (o / (Wo * Ho)) % d->M,
            n = o / (Wo * Ho * d->M);
    int64_t gm = m / (d->M / d->group);
    int64_t wz = w_zp ? (int64_t)w_zp[m] : 0;
    int64_t acc = bias_q ? (int64_t)bias_q[m] : 0;
    for (int64_t c = 0; c < cpg; ++c) {
      const int32_t* xplane = x + ((n * d->C) + gm * cpg + c) * d->H * d->W;
      const int32_t* wk = w + ((m * cpg) + c) * d->kH * d->kW;
      for (int64_t kh = 0; kh < d->kH; ++kh) {
        int64_t ih = oh * d->s_h - d->p_t + kh * d->d_h;
        if (ih < 0 || ih >= d->H) continue;
        for (int64_t kw = 0; kw < d->kW; ++kw) {
          int64_t iw = ow * d->s_w - d->p_l + kw * d->d_w;
          if (iw < 0 || iw >= d->W) continue;
          acc += ((int64_t)xplane[ih * d->W + iw] - x_zp) * ((int64_t)wk[kh * d->kW + kw] - wz);
        }
      }
    }
    if (acc >= INT32_LIMIT || acc < -INT32_LIMIT) bad = 1;
    if (acc_out) acc_out[o] = acc;
    if (y_out) y_out[o] = requant_range(acc, x_s, w_s[m], y_s, y_zp, y_lo, y_hi);
  }
  return bad ? OXREF_ERANGE : OXREF_OK;
}

int oxref_qgemm(int64_t M, int64_t N, int64_t K, const int32_t* x, const int32_t* w,
                const int32_t* bias_q, int32_t x_zp, const int32_t* w_zp, float x_s,
                const float* w_s, float y_s, int32_t y_zp, int32_t y_lo, int32_t y_hi,
                int64_t* acc_out, int32_t* y_out) {
  if (M < 0 || N < 0 || K < 0) return OXREF_EARG;
  if (!q_range_ok(y_zp, y_lo, y_hi)) return OXREF_EARG;
  if (M * N == 0) return OXREF_OK;
  if (K > 0 && (!x || !w)) return OXREF_EARG;
  if (y_out && !w_s) return OXREF_EARG;
  int bad = 0;
  int64_t total = M * N;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t o = 0; o < total; ++o) {
    int64_t i = o / N, j = o % N;
    int64_t wz = w_zp ? (int64_t)w_zp[j] : 0;
    int64_t acc = bias_q ? (int64_t)bias_q[j] : 0;
    for (int64_t k = 0; k < K; ++k)
      acc += ((int64_t)x[i * K + k] - x_zp) * ((int64_t)w[j * K + k] - wz);
    if (acc >= INT32_LIMIT || acc < -INT32_LIMIT) bad = 1;
    if (acc_out) acc_out[o] = acc;
    if (y_out) y_out[o] = requant_range(acc, x_s, w_s[j], y_s, y_zp, y_lo, y_hi);
  }
  return bad ? OXREF_ERANGE : OXREF_OK;
}
