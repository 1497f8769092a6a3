// ox_api.cpp -- the C ABI of libox: argument validation, kernel selection and
// the offline helpers.  Pure host code (no HIP runtime call happens before an
// argument set has passed validation), so every error path runs without a
// GPU.
//
// Validation is complete before anything is enqueued, and a refusal names the
// offending argument -- the load-time policy of onnx-vulkan-rs ("refuses at
// load time, naming every offender") applied per call.  An unsupported
// combination is refused, never approximated, and there is no CPU fallback
// (the OxiONNX 0.1.7 lesson: a quiet fallback hides a wrong answer).
//
// Selection follows "OxiONNX 0.1.7 Released" (Technical Deep Dive, items 2
// and 4): per shape, depthwise / 1x1 / implicit-GEMM for convolutions, a
// matrix-vector kernel for single-row Gemms, and the MFMA tile engine with a
// tile size chosen from the output shape for everything else.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "../../include/ox.h"
#include "ox_internal.h"

using namespace ox;

namespace {

thread_local std::string g_err;

ox_status fail(ox_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ox_status ok() {
  g_err.clear();
  return OX_OK;
}

ox_status hip_result(const char* fn, int rc) {
  if (rc != 0) return fail(OX_ERR_HIP, "%s: kernel launch failed (hip error %d)", fn, rc);
  return ok();
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;   // per tensor, exclusive

bool too_big(int64_t a, int64_t b = 1, int64_t c = 1, int64_t d = 1) {
  // product of non-negative factors >= 2^31, without overflowing
  long double p = (long double)a * b * c * d;
  return p >= (long double)kMaxElems;
}

int esize(int dt) { return dt == DT_F32 || dt == DT_I32 ? 4 : dt == DT_BF16 ? 2 : 1; }

bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

const char* act_name(int a) {
  static const char* n[] = {"none", "relu", "relu6", "gelu"};
  return (a >= 0 && a <= 3) ? n[a] : "?";
}

// OX_FORCE_KERNEL: comma-separated tokens, e.g. "igemm,tile=64x64".
struct Force {
  const char* variant = nullptr;   // "dw", "1x1", "pw", "patch", "smallc", "igemm", "gemv", "mfma"
  int tile = -1;
};

Force read_force() {
  Force f;
  static thread_local std::string buf;
  const char* e = getenv("OX_FORCE_KERNEL");
  if (!e || !*e) return f;
  buf = e;
  size_t pos = 0;
  static thread_local std::string variant;
  variant.clear();
  while (pos <= buf.size()) {
    size_t end = buf.find(',', pos);
    if (end == std::string::npos) end = buf.size();
    std::string tok = buf.substr(pos, end - pos);
    if (tok.rfind("tile=", 0) == 0) {
      for (int t = 0; t < TILE_COUNT; ++t)
        if (tok.substr(5) == tile_name(t)) f.tile = t;
      if (f.tile < 0) f.tile = -2;   // unknown tile name
    } else if (!tok.empty()) {
      variant = tok;
    }
    pos = end + 1;
  }
  if (!variant.empty()) f.variant = variant.c_str();
  return f;
}

bool log_on() {
  const char* e = getenv("OX_LOG");
  return e && *e && strcmp(e, "0") != 0;
}

// Tile choice: the largest tile that still gives two blocks per CU (the 256
// CUs of an MI355X), never a tile taller than the problem; a problem too
// small for that takes the smallest tile (the most blocks: each block's K
// loop, not the MMA rate, sets the time there).
int choose_tile(int64_t rows, int64_t cols, int64_t z) {
  static const int order[] = {TILE_128x128, TILE_64x128, TILE_128x64, TILE_64x64, TILE_32x64};
  for (int t : order) {
    const int bm = tile_bm(t), bn = tile_bn(t);
    if (rows <= 64 && bm > 64) continue;
    if (rows <= 32 && bm > 32) continue;
    // no 128-row tiles whose last row tile would be at most half full (its
    // blocks load as much as full ones for a fraction of the output):
    // MobileNetV2's 24->144 expands at 56², batch 64, bf16 34.8 -> 29.5 us
    // (64x128), fp32 58.8 -> 49.6 us; 32->192 at 28² fp32 24.1 -> 18.7 us
    if (bm == 128 && rows % 128 != 0 && rows % 128 <= 64) continue;
    const int64_t blocks = ((rows + bm - 1) / bm) * ((cols + bn - 1) / bn) * z;
    if (blocks >= 512) return t;
  }
  return TILE_32x64;
}

// Gemm / MatMul: the same rule without the 128x128 tile.  Their K loop keeps
// two stages in flight, whose registers would cost that tile an occupancy
// level (bf16 2048^3: 64x128 35.1 us against 38.1-52.7 us on 128x128).
int choose_tile_gemm(int64_t rows, int64_t cols, int64_t z) {
  static const int order[] = {TILE_64x128, TILE_128x64, TILE_64x64, TILE_32x64};
  for (int t : order) {
    const int bm = tile_bm(t), bn = tile_bn(t);
    if (rows <= 64 && bm > 64) continue;
    if (rows <= 32 && bm > 32) continue;
    const int64_t blocks = ((rows + bm - 1) / bm) * ((cols + bn - 1) / bn) * z;
    if (blocks >= 512) return t;
  }
  return TILE_32x64;
}

// fp32 implicit GEMM: every pixel column's elements are gathered one by one
// (offset arithmetic per element), so taller tiles (more output channels per
// gathered element) win, and 192 blocks already keep the chip busy through
// the long K.  Measured on ResNet-50's fp32 3x3 layers at batch 32 (us,
// against the generic rule): 64->64 at 56² 113.9 (145.7), 128 at 28² 111.6
// (134.6), 256 at 14² 140.0 (190.6), 512 at 7² 204.6 (211.5).
int choose_tile_igemm_f32(int64_t rows, int64_t cols, int64_t z) {
  static const int order[] = {TILE_128x64, TILE_64x64, TILE_32x64};
  for (int t : order) {
    const int bm = tile_bm(t), bn = tile_bn(t);
    if (rows <= 64 && bm > 64) continue;
    if (rows <= 32 && bm > 32) continue;
    const int64_t blocks = ((rows + bm - 1) / bm) * ((cols + bn - 1) / bn) * z;
    if (blocks >= 192) return t;
  }
  return TILE_32x64;
}

// fp32 1x1 with K >= 64: every column element is its own 4-byte load, and
// 64x64 (else 32x64) tiles from 256 blocks measured best (ResNet-50 batch 32,
// us against the generic rule: 256->64 at 56² 46.3 (59.5), 256->1024 at 14²
// 44.5 (52.5), 1024->256 at 14² 48.7 (50.9)); a K below 64 keeps the generic
// rule (16->96 at 112², output-bound: 128x128 99.2 against 64x64 113.1).
int choose_tile_1x1_f32(int64_t rows, int64_t cols, int64_t z) {
  static const int order[] = {TILE_64x64, TILE_32x64};
  for (int t : order) {
    const int bm = tile_bm(t), bn = tile_bn(t);
    if (rows <= 32 && bm > 32) continue;
    // (a last row tile at most half full: 32-row tiles waste nothing there;
    // MobileNetV2's 96-channel projections 21.9-28.4 us against 24.5-32.6)
    if (bm == 64 && rows % 64 != 0 && rows % 64 <= 32) continue;
    const int64_t blocks = ((rows + bm - 1) / bm) * ((cols + bn - 1) / bn) * z;
    if (blocks >= 256) return t;
  }
  return TILE_32x64;
}

enum TileRule { RULE_CONV = 0, RULE_GEMM = 1, RULE_IGEMM_F32 = 2, RULE_1X1_F32 = 3 };

ox_status pick_tile(const char* fn, const Force& f, int64_t rows, int64_t cols, int64_t z,
                    int* tile, int rule = RULE_CONV) {
  if (f.tile == -2) return fail(OX_ERR_INVALID_ARG, "%s: OX_FORCE_KERNEL names an unknown tile", fn);
  *tile = f.tile >= 0 ? f.tile
          : rule == RULE_GEMM ? choose_tile_gemm(rows, cols, z)
          : rule == RULE_IGEMM_F32 ? choose_tile_igemm_f32(rows, cols, z)
          : rule == RULE_1X1_F32 ? choose_tile_1x1_f32(rows, cols, z)
                                 : choose_tile(rows, cols, z);
  if ((rows + tile_bm(*tile) - 1) / tile_bm(*tile) > 65535 || z > 65535)
    return fail(OX_ERR_UNSUPPORTED, "%s: %lld rows x batch %lld exceed the launch grid", fn,
                (long long)rows, (long long)z);
  return OX_OK;
}

ox_status check_float_dt(const char* fn, ox_dtype t) {
  if (t != OX_F32 && t != OX_BF16)
    return fail(OX_ERR_UNSUPPORTED, "%s: dtype %d is not OX_F32 or OX_BF16", fn, (int)t);
  return OX_OK;
}

ox_status check_act(const char* fn, ox_act a) {
  if ((int)a < 0 || (int)a > 3) return fail(OX_ERR_INVALID_ARG, "%s: unknown activation %d", fn, (int)a);
  return OX_OK;
}

// ---------------------------------------------------------------- conv ----

ox_status check_conv_desc(const char* fn, const ox_conv_desc* d, int64_t* Ho, int64_t* Wo) {
  if (!d) return fail(OX_ERR_INVALID_ARG, "%s: d is NULL", fn);
  if (d->N < 0) return fail(OX_ERR_INVALID_ARG, "%s: N=%lld < 0", fn, (long long)d->N);
  const struct { const char* n; int64_t v; } pos[] = {
      {"C", d->C}, {"H", d->H}, {"W", d->W}, {"M", d->M}, {"kH", d->kH}, {"kW", d->kW},
      {"s_h", d->s_h}, {"s_w", d->s_w}, {"d_h", d->d_h}, {"d_w", d->d_w}, {"group", d->group}};
  for (auto& p : pos)
    if (p.v < 1) return fail(OX_ERR_INVALID_ARG, "%s: %s=%lld must be >= 1", fn, p.n, (long long)p.v);
  const struct { const char* n; int64_t v; } pads[] = {
      {"p_t", d->p_t}, {"p_l", d->p_l}, {"p_b", d->p_b}, {"p_r", d->p_r}};
  for (auto& p : pads)
    if (p.v < 0) return fail(OX_ERR_INVALID_ARG, "%s: %s=%lld must be >= 0", fn, p.n, (long long)p.v);
  if (d->C % d->group)
    return fail(OX_ERR_SHAPE, "%s: group=%lld does not divide C=%lld", fn, (long long)d->group,
                (long long)d->C);
  if (d->M % d->group)
    return fail(OX_ERR_SHAPE, "%s: group=%lld does not divide M=%lld", fn, (long long)d->group,
                (long long)d->M);
  const int64_t lim = (int64_t)1 << 24;   // geometry limits keep kernel index math in int32
  if (d->H >= lim || d->W >= lim || d->kH >= lim || d->kW >= lim || d->s_h >= lim ||
      d->s_w >= lim || d->d_h >= lim || d->d_w >= lim || d->p_t >= lim || d->p_l >= lim ||
      d->p_b >= lim || d->p_r >= lim)
    return fail(OX_ERR_UNSUPPORTED, "%s: a size, stride, pad or dilation is >= 2^24", fn);
  const int64_t eh = d->d_h * (d->kH - 1) + 1, ew = d->d_w * (d->kW - 1) + 1;
  const int64_t sh = d->H + d->p_t + d->p_b - eh, sw = d->W + d->p_l + d->p_r - ew;
  *Ho = sh < 0 ? 0 : sh / d->s_h + 1;
  *Wo = sw < 0 ? 0 : sw / d->s_w + 1;
  if (*Ho < 1 || *Wo < 1)
    return fail(OX_ERR_SHAPE,
                "%s: output size %lldx%lld < 1 (input %lldx%lld, pads %lld,%lld,%lld,%lld, "
                "dilated kernel %lldx%lld)",
                fn, (long long)*Ho, (long long)*Wo, (long long)d->H, (long long)d->W,
                (long long)d->p_t, (long long)d->p_l, (long long)d->p_b, (long long)d->p_r,
                (long long)eh, (long long)ew);
  if (too_big(d->N, d->C, d->H, d->W)) return fail(OX_ERR_UNSUPPORTED, "%s: X has >= 2^31 elements", fn);
  if (too_big(d->M, d->C / d->group, d->kH, d->kW))
    return fail(OX_ERR_UNSUPPORTED, "%s: W has >= 2^31 elements", fn);
  if (too_big(d->N, d->M, *Ho, *Wo)) return fail(OX_ERR_UNSUPPORTED, "%s: Y has >= 2^31 elements", fn);
  return OX_OK;
}

ConvArgs conv_args(int dt, const ox_conv_desc* d, int64_t Ho, int64_t Wo, const void* X,
                   const void* W, const void* bias, void* Y, int act) {
  ConvArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = dt;
  a.out_dt = dt;
  a.N = (int)d->N;
  a.C = (int)d->C;
  a.H = (int)d->H;
  a.W = (int)d->W;
  a.M = (int)d->M;
  a.kH = (int)d->kH;
  a.kW = (int)d->kW;
  a.sh = (int)d->s_h;
  a.sw = (int)d->s_w;
  a.pt = (int)d->p_t;
  a.pl = (int)d->p_l;
  a.dh = (int)d->d_h;
  a.dw = (int)d->d_w;
  a.group = (int)d->group;
  a.Ho = (int)Ho;
  a.Wo = (int)Wo;
  a.X = X;
  a.Wt = W;
  a.bias = bias;
  a.Y = Y;
  a.act = act;
  const int64_t K = (d->C / d->group) * d->kH * d->kW;
  a.w_vec = aligned16(W) && (K * esize(dt)) % 16 == 0;
  a.x_vec = aligned16(X) && (d->H * d->W * esize(dt)) % 16 == 0;
  return a;
}

enum ConvKind { KIND_IGEMM = 0, KIND_1X1 = 1, KIND_DW = 2, KIND_PATCH = 3, KIND_PW = 4, KIND_SMALLC = 5,
                KIND_PWD = 6, KIND_DWR = 7 };

const char* kind_name(int k) {
  static const char* n[] = {"igemm", "1x1", "dw", "patch", "pw", "smallc", "pwd", "dwr"};
  return n[k];
}

// The DMA pointwise kernel where it applies, unless the input channels are
// not a multiple of 64 and the layer has fewer than 65536 pixels: there (32
// or 96 channels into a few thousand pixels: MobileNetV2's narrow expand
// layers) the register-staged kernel was 10-45% faster in the per-layer A/B
// runs, while with many pixels (its 96 -> 24 projection at 56x56) the DMA
// kernel stayed 12% ahead.
bool pwd_preferred(const ConvArgs& a) {
  return (a.C % 64 == 0 || (int64_t)a.N * a.H * a.W >= 65536) && conv_pwd_applicable(a);
}

// The register-staged 1x1 kernel, except on an odd plane with a short K or
// few output channels: its channel runs are then single pixels and the tile
// engine's kernel (buffer loaders, one 2-byte element per load) is faster
// (MobileNetV2 at 7x7: 160->960 16.2 -> 10.3 us, 576->160 15.6 -> 9.2,
// 960->160 17.7 -> 12.8, 960->320 22.4 -> 17.2; ResNet-50's 2048->512 stays
// on pw: 24.1 against 30.7).
bool pw_preferred(const ConvArgs& a) {
  return !((a.H * a.W) % 2 == 1 && (a.C <= 192 || a.M <= 384)) && conv_pw_applicable(a);
}

ox_status select_conv(const char* fn, const ox_conv_desc* d, const ConvArgs& a, const Force& f,
                      int* kind) {
  if (a.w_packed) {
    // packed weights exist only for the LDS-patch kernel (which takes no residual)
    if (a.res)
      return fail(OX_ERR_UNSUPPORTED, "%s: packed weights do not take a residual input", fn);
    if (f.variant && strcmp(f.variant, "patch"))
      return fail(OX_ERR_UNSUPPORTED, "%s: OX_FORCE_KERNEL variant '%s' does not take packed weights", fn,
                  f.variant);
    if (!conv_patch_applicable(a))
      return fail(OX_ERR_UNSUPPORTED,
                  "%s: no packed-weight kernel for this geometry or alignment (needs bf16, 3x3, group 1, "
                  "C %% 32 == 0, stride 1 or 2, 16-byte aligned X and W)", fn);
    *kind = KIND_PATCH;
    return OX_OK;
  }
  const bool is_dw = d->group == d->C && d->group == d->M;
  const bool is_1x1 = d->kH == 1 && d->kW == 1 && d->s_h == 1 && d->s_w == 1 && d->p_t == 0 &&
                      d->p_l == 0 && d->p_b == 0 && d->p_r == 0 && d->group == 1;
  if (f.variant) {
    if (!strcmp(f.variant, "dwr")) {
      if (!is_dw || !depthwise_rows_applicable(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'dwr' needs a 3x3 depthwise conv with pads 1, stride 1 or 2, "
                    "fp32 or bf16, an even W (bf16 or stride 2), Wo <= 512 and 4-byte aligned X", fn);
      *kind = KIND_DWR;
    } else if (!strcmp(f.variant, "dw")) {
      if (!is_dw) return fail(OX_ERR_UNSUPPORTED, "%s: forced 'dw' but group != C or C != M", fn);
      if (!depthwise_fits(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'dw' but the row band does not fit LDS", fn);
      *kind = KIND_DW;
    } else if (!strcmp(f.variant, "1x1")) {
      if (!is_1x1) return fail(OX_ERR_UNSUPPORTED, "%s: forced '1x1' on a conv that is not 1x1/s1/p0/g1", fn);
      *kind = KIND_1X1;
    } else if (!strcmp(f.variant, "pw")) {
      if (!is_1x1 || !conv_pw_applicable(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'pw' needs bf16, a 1x1/s1/p0/g1 conv, C %% 32 == 0 and aligned X/W", fn);
      *kind = KIND_PW;
    } else if (!strcmp(f.variant, "pwd")) {
      if (!is_1x1 || !conv_pwd_applicable(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'pwd' needs bf16, a 1x1/s1/p0/g1 conv, C %% 32 == 0, "
                    "H*W %% 8 == 0 and 16-byte aligned X/W/Y", fn);
      *kind = KIND_PWD;
    } else if (!strcmp(f.variant, "smallc")) {
      if (!conv_smallc_applicable(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'smallc' needs bf16, C <= 4, group 1, stride 1 or 2, no dilation, kW <= 8", fn);
      *kind = KIND_SMALLC;
    } else if (!strcmp(f.variant, "igemm")) {
      *kind = KIND_IGEMM;
    } else if (!strcmp(f.variant, "patch")) {
      if (!conv_patch_applicable(a))
        return fail(OX_ERR_UNSUPPORTED, "%s: forced 'patch' needs bf16, a 3x3 kernel, group 1, C %% 32 == 0 and aligned X/W", fn);
      *kind = KIND_PATCH;
    } else {
      return fail(OX_ERR_INVALID_ARG, "%s: OX_FORCE_KERNEL variant '%s' does not apply to Conv", fn,
                  f.variant);
    }
    if (a.res && *kind != KIND_PW && *kind != KIND_PWD && *kind != KIND_1X1 && *kind != KIND_IGEMM)
      return fail(OX_ERR_UNSUPPORTED, "%s: forced '%s' does not take a residual input", fn, f.variant);
    return OX_OK;
  }
  if (a.res) {
    // a residual input: the kernels whose epilogue reads it are the
    // pointwise kernel and the tile engine (any geometry)
    if (is_1x1) *kind = pwd_preferred(a) ? KIND_PWD : pw_preferred(a) ? KIND_PW : KIND_1X1;
    else *kind = KIND_IGEMM;
    return OX_OK;
  }
  if (is_dw && depthwise_rows_applicable(a)) *kind = KIND_DWR;
  else if (is_dw && depthwise_fits(a)) *kind = KIND_DW;
  else if (is_1x1) *kind = pwd_preferred(a) ? KIND_PWD : pw_preferred(a) ? KIND_PW : KIND_1X1;
  else if (conv_patch_applicable(a)) *kind = KIND_PATCH;
  else if (conv_smallc_applicable(a)) *kind = KIND_SMALLC;
  else *kind = KIND_IGEMM;
  return OX_OK;
}

}  // namespace

// The stream-aware body of the convolution entry points.  static_ws: the
// workspace is the library's static scratch array (a plan needing more is
// refused as unsupported, not as a caller error).
static ox_status conv_dispatch(const char* fn, const ox_conv_desc* d, ConvArgs& a, void* stream,
                               bool static_ws = false) {
  const Force f = read_force();
  int kind;
  ox_status st = select_conv(fn, d, a, f, &kind);
  if (st) return st;
  int tile = -1;
  if (kind == KIND_IGEMM || kind == KIND_1X1) {
    st = pick_tile(fn, f, d->M / d->group, d->N * a.Ho * a.Wo, d->group, &tile,
                   a.dt != DT_F32 ? RULE_CONV : kind == KIND_IGEMM ? RULE_IGEMM_F32
                   : d->C / d->group >= 64 ? RULE_1X1_F32 : RULE_CONV);
    if (st) return st;
  } else if (f.tile != -1) {
    return fail(OX_ERR_INVALID_ARG, "%s: a tile does not apply to the %s kernel", fn, kind_name(kind));
  }
  if (a.ws) {
    const size_t need = kind == KIND_PW ? conv_pw_ws_bytes(a) : kind == KIND_PATCH ? conv_patch_ws_bytes(a) : 0;
    if (need > a.ws_bytes && static_ws)
      return fail(OX_ERR_UNSUPPORTED, "%s: this geometry's split-K plan needs %zu bytes of scratch, more than "
                  "the %zu of the static scratch array", fn, need, a.ws_bytes);
    if (need > a.ws_bytes)
      return fail(OX_ERR_INVALID_ARG, "%s: workspace_bytes=%zu < %zu that this geometry needs", fn,
                  a.ws_bytes, need);
  }
  if (log_on()) {
    char plan[160] = "";
    if (kind == KIND_PATCH) conv_patch_describe(a, plan, sizeof(plan));
    if (kind == KIND_PW) conv_pw_describe(a, plan, sizeof(plan));
    if (kind == KIND_PWD) conv_pwd_describe(a, plan, sizeof(plan));
    if (kind == KIND_DWR) conv_depthwise_rows_describe(a, plan, sizeof(plan));
    if (kind == KIND_SMALLC) conv_smallc_describe(a, plan, sizeof(plan));
    fprintf(stderr, "[ox] %s dt=%d N=%d C=%d %dx%d M=%d k=%dx%d s=%d,%d g=%d act=%s -> %s%s%s %s\n",
            fn, a.dt, a.N, a.C, a.H, a.W, a.M, a.kH, a.kW, a.sh, a.sw, a.group, act_name(a.act),
            kind_name(kind), tile >= 0 ? " tile=" : "", tile >= 0 ? tile_name(tile) : "", plan);
  }
  if (d->N == 0) return ok();
  int rc;
  if (kind == KIND_DW) {
    rc = launch_conv_depthwise(a, stream);
  } else if (kind == KIND_DWR) {
    rc = launch_conv_depthwise_rows(a, stream);
  } else if (kind == KIND_PATCH) {
    rc = launch_conv_patch(a, stream);
  } else if (kind == KIND_PW) {
    rc = launch_conv_pw(a, stream);
  } else if (kind == KIND_PWD) {
    rc = launch_conv_pwd(a, stream);
  } else if (kind == KIND_SMALLC) {
    rc = launch_conv_smallc(a, stream);
  } else {
    const int k = kind == KIND_1X1 ? 1 : 0;
    rc = a.dt == DT_F32 ? launch_conv_f32(a, k, tile, stream)
       : a.dt == DT_BF16 ? launch_conv_bf16(a, k, tile, stream)
                         : launch_conv_i8(a, k, tile, stream);
  }
  return hip_result(fn, rc);
}

// ------------------------------------------------------------------ API ----

extern "C" {

const char* ox_last_error(void) { return g_err.c_str(); }

const char* ox_version(void) { return "ox 0.1.0 (gfx950)"; }

ox_status ox_matmul_batched(ox_dtype t, int64_t batch, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t sA, const void* B, int64_t sB, void* C,
                            void* stream) {
  const char* fn = "ox_matmul_batched";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  if (batch < 0 || M < 0 || N < 0 || K < 0)
    return fail(OX_ERR_INVALID_ARG, "%s: negative size (batch=%lld M=%lld N=%lld K=%lld)", fn,
                (long long)batch, (long long)M, (long long)N, (long long)K);
  if (batch > 1 && sA < M * K)
    return fail(OX_ERR_INVALID_ARG, "%s: sA=%lld < M*K=%lld", fn, (long long)sA, (long long)(M * K));
  if (batch > 1 && sB != 0 && sB < K * N)
    return fail(OX_ERR_INVALID_ARG, "%s: sB=%lld is neither 0 (broadcast) nor >= K*N=%lld", fn,
                (long long)sB, (long long)(K * N));
  if (sA < 0 || sB < 0) return fail(OX_ERR_INVALID_ARG, "%s: negative batch stride", fn);
  if (too_big(M, K) || too_big(K, N) || too_big(batch, M, N) ||
      (batch > 1 && (too_big(sA, batch) || too_big(sB, batch))))
    return fail(OX_ERR_UNSUPPORTED, "%s: a tensor has >= 2^31 elements", fn);
  if (batch == 0 || M == 0 || N == 0) return ok();
  if (!C) return fail(OX_ERR_INVALID_ARG, "%s: C is NULL", fn);
  if (K > 0 && (!A || !B)) return fail(OX_ERR_INVALID_ARG, "%s: %s is NULL", fn, A ? "B" : "A");
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = a.out_dt = (int)t;
  a.rows = (int)M;
  a.cols = (int)N;
  a.K = (int)K;
  a.batch = (int)batch;
  a.L = A;
  a.ldl = K;
  a.sl = sA;
  a.l_kmajor = 1;
  a.R = B;
  a.ldr = N;
  a.sr = sB;
  a.r_kmajor = 0;
  a.Y = C;
  a.ldy = N;
  a.sy = M * N;
  a.alpha = 1.0f;
  a.beta = 0.0f;
  a.act = ACT_NONE;
  const int es = esize(t);
  a.l_vec = aligned16(A) && (K * es) % 16 == 0 && (sA * es) % 16 == 0;
  a.r_vec = 0;
  const Force f = read_force();
  if (f.variant && strcmp(f.variant, "mfma"))
    return fail(OX_ERR_UNSUPPORTED, "%s: OX_FORCE_KERNEL variant '%s' does not apply to MatMul", fn,
                f.variant);
  int tile;
  st = pick_tile(fn, f, M, N, batch, &tile, RULE_GEMM);
  if (st) return st;
  if (log_on())
    fprintf(stderr, "[ox] %s dt=%d batch=%lld M=%lld N=%lld K=%lld sB=%lld -> mfma tile=%s\n", fn,
            (int)t, (long long)batch, (long long)M, (long long)N, (long long)K, (long long)sB,
            tile_name(tile));
  const int rc = t == OX_F32 ? launch_gemm_f32(a, tile, stream) : launch_gemm_bf16(a, tile, stream);
  return hip_result(fn, rc);
}

// Split-K plan of a float Gemm: 0 when none.  Only problems that no tile
// fills the chip with (they take 32x64 tiles, here fewer than 256 of them)
// and whose K gives every slice at least four deep stages; at most 8 slices
// and about one block per CU.
struct GemmSplit {
  int S, kslice;
};
static GemmSplit gemm_split_plan(ox_dtype t, int64_t M, int64_t N, int64_t K) {
  GemmSplit g = {0, 0};
  if (t != OX_F32 && t != OX_BF16) return g;
  if (M <= 1 || N <= 0 || K <= 0) return g;
  if (choose_tile_gemm(M, N, 1) != TILE_32x64) return g;
  const int64_t blocks = ((M + 31) / 32) * ((N + 63) / 64);
  if (blocks >= 256) return g;
  const int64_t kstep = t == OX_F32 ? 64 : 128;   // four 64-byte units per stage
  const int64_t stages = (K + kstep - 1) / kstep;
  // below 64 units the single pass (two stages in flight) wins: bf16 M = 64 /
  // 256, K = 1024: 7.7 / 7.8 us against 8.5 / 9.2 us split
  if (stages < 16) return g;
  int64_t S = std::min<int64_t>({8, 256 / blocks, stages / 4});
  if (S < 2) return g;
  const int64_t kslice = (stages + S - 1) / S * kstep;
  S = (K + kslice - 1) / kslice;
  if (S < 2) return g;
  g.S = (int)S;
  g.kslice = (int)kslice;
  return g;
}

size_t ox_gemm_workspace_bytes(ox_dtype t, int64_t M, int64_t N, int64_t K) {
  const GemmSplit g = gemm_split_plan(t, M, N, K);
  return g.S ? (size_t)g.S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

static ox_status gemm_fused_impl(const char* fn, ox_dtype t, int64_t M, int64_t N, int64_t K,
                                 int transA, int transB, float alpha, const void* A, const void* B,
                                 float beta, const void* bias, ox_act act, void* Y,
                                 const void* int8_params, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const bool i8 = t == OX_I8 || t == OX_I32;
  if (!i8) {
    ox_status st = check_float_dt(fn, t);
    if (st) return st;
  }
  ox_status st = check_act(fn, act);
  if (st) return st;
  if (M < 0 || N < 0 || K < 0)
    return fail(OX_ERR_INVALID_ARG, "%s: negative size (M=%lld N=%lld K=%lld)", fn, (long long)M,
                (long long)N, (long long)K);
  if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1))
    return fail(OX_ERR_INVALID_ARG, "%s: transA/transB must be 0 or 1", fn);
  if (!isfinite(alpha) || !isfinite(beta))
    return fail(OX_ERR_INVALID_ARG, "%s: alpha and beta must be finite", fn);
  if (too_big(M, K) || too_big(K, N) || too_big(M, N))
    return fail(OX_ERR_UNSUPPORTED, "%s: a tensor has >= 2^31 elements", fn);
  if (i8) {
    if (transA != 0 || transB != 1)
      return fail(OX_ERR_UNSUPPORTED, "%s: int8 Gemm needs transA=0 and transB=1 (W stored [N,K])", fn);
    if (bias) return fail(OX_ERR_INVALID_ARG, "%s: int8 Gemm takes its int32 bias in int8_params; bias must be NULL", fn);
    if (alpha != 1.0f || beta != 1.0f)
      return fail(OX_ERR_UNSUPPORTED, "%s: int8 Gemm needs alpha = beta = 1", fn);
    if (act != OX_ACT_NONE) return fail(OX_ERR_UNSUPPORTED, "%s: int8 Gemm takes no activation", fn);
    if (!int8_params) return fail(OX_ERR_INVALID_ARG, "%s: int8_params is NULL", fn);
  } else if (int8_params) {
    return fail(OX_ERR_INVALID_ARG, "%s: int8_params must be NULL for a float Gemm", fn);
  }
  if (M == 0 || N == 0) return ok();
  if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  if (K > 0 && (!A || !B)) return fail(OX_ERR_INVALID_ARG, "%s: %s is NULL", fn, A ? "B" : "A");

  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = i8 ? DT_I8 : (int)t;
  a.out_dt = (int)t;
  a.rows = (int)M;
  a.cols = (int)N;
  a.K = (int)K;
  a.batch = 1;
  a.L = A;
  a.l_kmajor = transA ? 0 : 1;
  a.ldl = transA ? M : K;
  a.R = B;
  a.r_kmajor = transB ? 1 : 0;
  a.ldr = transB ? K : N;
  a.Y = Y;
  a.ldy = N;
  a.bias = bias;
  a.alpha = alpha;
  a.beta = beta;
  a.act = (int)act;
  a.i8 = int8_params;
  const int es = esize(a.dt);
  a.l_vec = aligned16(A) && (a.ldl * es) % 16 == 0;
  a.r_vec = aligned16(B) && (a.ldr * es) % 16 == 0;

  const Force f = read_force();
  bool gemv = !i8 && M == 1;
  if (f.variant) {
    if (!strcmp(f.variant, "gemv")) {
      if (i8 || M != 1) return fail(OX_ERR_UNSUPPORTED, "%s: forced 'gemv' needs a float Gemm with M=1", fn);
      gemv = true;
    } else if (!strcmp(f.variant, "mfma")) {
      gemv = false;
    } else {
      return fail(OX_ERR_INVALID_ARG, "%s: OX_FORCE_KERNEL variant '%s' does not apply to Gemm", fn,
                  f.variant);
    }
  }
  if (gemv) {
    if (f.tile != -1) return fail(OX_ERR_INVALID_ARG, "%s: a tile does not apply to gemv", fn);
    if (log_on())
      fprintf(stderr, "[ox] %s dt=%d M=1 N=%lld K=%lld transB=%d act=%s -> gemv\n", fn, (int)t,
              (long long)N, (long long)K, transB, act_name(act));
    return hip_result(fn, launch_gemv(a, stream));
  }
  if (workspace && !i8 && f.tile == -1) {
    const GemmSplit g = gemm_split_plan(t, M, N, K);
    if (g.S) {
      const size_t need = (size_t)g.S * (size_t)M * (size_t)N * sizeof(float);
      if (workspace_bytes < need || (uintptr_t)workspace % 16)
        return fail(OX_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned and hold %zu bytes", fn,
                    need);
      if (log_on())
        fprintf(stderr, "[ox] %s dt=%d M=%lld N=%lld K=%lld -> mfma split-K S=%d kslice=%d\n", fn,
                (int)t, (long long)M, (long long)N, (long long)K, g.S, g.kslice);
      const int rc = t == OX_F32 ? launch_gemm_splitk_f32(a, g.S, g.kslice, (float*)workspace, stream)
                                 : launch_gemm_splitk_bf16(a, g.S, g.kslice, (float*)workspace, stream);
      return hip_result(fn, rc);
    }
  }
  int tile;
  st = pick_tile(fn, f, M, N, 1, &tile, RULE_GEMM);
  if (st) return st;
  if (log_on())
    fprintf(stderr, "[ox] %s dt=%d M=%lld N=%lld K=%lld tA=%d tB=%d act=%s -> mfma tile=%s\n", fn,
            (int)t, (long long)M, (long long)N, (long long)K, transA, transB, act_name(act),
            tile_name(tile));
  const int rc = i8 ? launch_gemm_i8(a, tile, stream)
               : t == OX_F32 ? launch_gemm_f32(a, tile, stream)
                             : launch_gemm_bf16(a, tile, stream);
  return hip_result(fn, rc);
}

ox_status ox_gemm_fused(ox_dtype t, int64_t M, int64_t N, int64_t K, int transA, int transB,
                        float alpha, const void* A, const void* B, float beta, const void* bias,
                        ox_act act, void* Y, const void* int8_params, void* stream) {
  return gemm_fused_impl("ox_gemm_fused", t, M, N, K, transA, transB, alpha, A, B, beta, bias, act,
                         Y, int8_params, nullptr, 0, stream);
}

ox_status ox_gemm_fused_ws(ox_dtype t, int64_t M, int64_t N, int64_t K, int transA, int transB,
                           float alpha, const void* A, const void* B, float beta, const void* bias,
                           ox_act act, void* Y, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (t != OX_F32 && t != OX_BF16)
    return fail(OX_ERR_UNSUPPORTED, "ox_gemm_fused_ws: dtype %d is not OX_F32 or OX_BF16", (int)t);
  return gemm_fused_impl("ox_gemm_fused_ws", t, M, N, K, transA, transB, alpha, A, B, beta, bias,
                         act, Y, nullptr, workspace, workspace_bytes, stream);
}

ox_status ox_conv2d_fused(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                          const void* bias, ox_act act, void* Y, void* stream) {
  const char* fn = "ox_conv2d_fused";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  st = check_act(fn, act);
  if (st) return st;
  int64_t Ho, Wo;
  st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  if (d->N > 0) {
    if (!X) return fail(OX_ERR_INVALID_ARG, "%s: X is NULL", fn);
    if (!W) return fail(OX_ERR_INVALID_ARG, "%s: W is NULL", fn);
    if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  }
  ConvArgs a = conv_args((int)t, d, Ho, Wo, X, W, bias, Y, (int)act);
  return conv_dispatch(fn, d, a, stream);
}

size_t ox_conv2d_packed_weights_bytes(ox_dtype t, const ox_conv_desc* d) {
  int64_t Ho, Wo;
  if ((t != OX_F32 && t != OX_BF16) || check_conv_desc("ox_conv2d_packed_weights_bytes", d, &Ho, &Wo))
    return 0;
  ConvArgs a = conv_args((int)t, d, Ho, Wo, nullptr, nullptr, nullptr, nullptr, ACT_NONE);
  if (!conv_patch_geometry(a)) return 0;
  return (size_t)(d->M * d->C * d->kH * d->kW) * esize(t);
}

ox_status ox_conv2d_pack_weights(ox_dtype t, const ox_conv_desc* d, const void* W_host, void* Wp_host) {
  const char* fn = "ox_conv2d_pack_weights";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  int64_t Ho, Wo;
  st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  ConvArgs a = conv_args((int)t, d, Ho, Wo, nullptr, nullptr, nullptr, nullptr, ACT_NONE);
  if (!conv_patch_geometry(a))
    return fail(OX_ERR_UNSUPPORTED, "%s: no packed layout for this geometry (needs bf16, 3x3, group 1, "
                "C %% 32 == 0, stride 1 or 2)", fn);
  if (!W_host || !Wp_host) return fail(OX_ERR_INVALID_ARG, "%s: W_host or Wp_host is NULL", fn);
  const int64_t M = d->M, Cc = d->C, KK = d->kH * d->kW, nch = Cc / 32;
  const int es = esize(t);
  const char* src = (const char*)W_host;
  char* dst = (char*)Wp_host;
  // Wp[m][chunk][tap][c32] = W[m][chunk*32 + c32][tap]
  for (int64_t m = 0; m < M; ++m)
    for (int64_t ch = 0; ch < nch; ++ch)
      for (int64_t tap = 0; tap < KK; ++tap)
        for (int64_t c = 0; c < 32; ++c)
          memcpy(dst + (((m * nch + ch) * KK + tap) * 32 + c) * es,
                 src + ((m * Cc + ch * 32 + c) * KK + tap) * es, es);
  return ok();
}

ox_status ox_conv2d_fused_packed(ox_dtype t, const ox_conv_desc* d, const void* X, const void* Wp,
                                 const void* bias, ox_act act, void* Y, void* stream) {
  const char* fn = "ox_conv2d_fused_packed";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  st = check_act(fn, act);
  if (st) return st;
  int64_t Ho, Wo;
  st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  if (d->N > 0) {
    if (!X) return fail(OX_ERR_INVALID_ARG, "%s: X is NULL", fn);
    if (!Wp) return fail(OX_ERR_INVALID_ARG, "%s: Wp is NULL", fn);
    if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  }
  ConvArgs a = conv_args((int)t, d, Ho, Wo, X, Wp, bias, Y, (int)act);
  a.w_packed = 1;
  return conv_dispatch(fn, d, a, stream);
}

size_t ox_conv2d_workspace_bytes(ox_dtype t, const ox_conv_desc* d) {
  const char* fn = "ox_conv2d_workspace_bytes";
  int64_t Ho, Wo;
  if ((t != OX_F32 && t != OX_BF16) || check_conv_desc(fn, d, &Ho, &Wo)) return 0;
  ConvArgs a = conv_args((int)t, d, Ho, Wo, nullptr, nullptr, nullptr, nullptr, ACT_NONE);
  a.ws = (void*)(uintptr_t)256;   // "a workspace will be given": plan with split-K allowed
  a.ws_bytes = SIZE_MAX;
  const Force f = read_force();
  int kind;
  if (select_conv(fn, d, a, f, &kind)) return 0;
  return kind == KIND_PW ? conv_pw_ws_bytes(a) : kind == KIND_PATCH ? conv_patch_ws_bytes(a) : 0;
}

static ox_status conv_fused_ws_res(const char* fn, ox_dtype t, const ox_conv_desc* d, const void* X,
                                   const void* W, int w_packed, const void* bias, const void* R,
                                   ox_act act, void* Y, void* workspace, size_t workspace_bytes,
                                   void* stream, bool static_ws = false) {
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  st = check_act(fn, act);
  if (st) return st;
  if (w_packed != 0 && w_packed != 1) return fail(OX_ERR_INVALID_ARG, "%s: w_packed=%d is not 0 or 1", fn, w_packed);
  if (workspace && ((uintptr_t)workspace) % 16)
    return fail(OX_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  if (R && ((uintptr_t)R) % (t == OX_F32 ? 4 : 2))
    return fail(OX_ERR_INVALID_ARG, "%s: R is not aligned to its element size", fn);
  int64_t Ho, Wo;
  st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  if (d->N > 0) {
    if (!X) return fail(OX_ERR_INVALID_ARG, "%s: X is NULL", fn);
    if (!W) return fail(OX_ERR_INVALID_ARG, "%s: W is NULL", fn);
    if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  }
  ConvArgs a = conv_args((int)t, d, Ho, Wo, X, W, bias, Y, (int)act);
  a.w_packed = w_packed;
  a.ws = workspace;
  a.ws_bytes = workspace ? workspace_bytes : 0;
  a.res = R;
  if (static_ws) {
    // the static array's address on this device, only now that every
    // argument has passed (a refused call makes no HIP call at all)
    const Force f = read_force();
    int kind;
    st = select_conv(fn, d, a, f, &kind);
    if (st) return st;
    const size_t need = kind == KIND_PW ? conv_pw_ws_bytes(a) : kind == KIND_PATCH ? conv_patch_ws_bytes(a) : 0;
    if (need > workspace_bytes)
      return fail(OX_ERR_UNSUPPORTED, "%s: this geometry's split-K plan needs %zu bytes of scratch, more "
                  "than the %zu of the static scratch array", fn, need, workspace_bytes);
    void* p = nullptr;
    const int rc = static_scratch(&p);
    if (rc) return fail(OX_ERR_HIP, "%s: looking up the static scratch array failed (hip error %d)", fn, rc);
    a.ws = p;
  }
  return conv_dispatch(fn, d, a, stream, static_ws);
}

size_t ox_static_scratch_bytes(void) { return static_scratch_bytes(); }

ox_status ox_conv2d_fused_static(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                                 int w_packed, const void* bias, ox_act act, void* Y, void* stream) {
  // a non-null stand-in until the arguments are checked; replaced by the
  // device address of the static array before anything is enqueued
  return conv_fused_ws_res("ox_conv2d_fused_static", t, d, X, W, w_packed, bias, nullptr, act, Y,
                           (void*)(uintptr_t)256, static_scratch_bytes(), stream, true);
}

ox_status ox_conv2d_fused_ws(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                             int w_packed, const void* bias, ox_act act, void* Y, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return conv_fused_ws_res("ox_conv2d_fused_ws", t, d, X, W, w_packed, bias, nullptr, act, Y, workspace,
                           workspace_bytes, stream);
}

ox_status ox_conv2d_fused_res(ox_dtype t, const ox_conv_desc* d, const void* X, const void* W,
                              const void* bias, const void* R, ox_act act, void* Y, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return conv_fused_ws_res("ox_conv2d_fused_res", t, d, X, W, 0, bias, R, act, Y, workspace,
                           workspace_bytes, stream);
}

ox_status ox_conv2d_int8(const ox_conv_desc* d, const int8_t* Xq, const int8_t* Wq,
                         const void* int8_params, ox_dtype y_type, void* Y, void* stream) {
  const char* fn = "ox_conv2d_int8";
  if (y_type != OX_I8 && y_type != OX_I32)
    return fail(OX_ERR_UNSUPPORTED, "%s: y_type %d is not OX_I8 or OX_I32", fn, (int)y_type);
  int64_t Ho, Wo;
  ox_status st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  if (!int8_params) return fail(OX_ERR_INVALID_ARG, "%s: int8_params is NULL", fn);
  if (d->N > 0) {
    if (!Xq) return fail(OX_ERR_INVALID_ARG, "%s: Xq is NULL", fn);
    if (!Wq) return fail(OX_ERR_INVALID_ARG, "%s: Wq is NULL", fn);
    if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  }
  ConvArgs a = conv_args(DT_I8, d, Ho, Wo, Xq, Wq, nullptr, Y, ACT_NONE);
  a.out_dt = (int)y_type;
  a.i8 = int8_params;
  return conv_dispatch(fn, d, a, stream);
}

ox_status ox_batchnorm_act(ox_dtype t, int64_t N, int64_t C, int64_t HW, const void* X,
                           const float* gamma, const float* beta, const float* mean, const float* var,
                           float eps, ox_act act, void* Y, void* stream) {
  const char* fn = "ox_batchnorm_act";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  st = check_act(fn, act);
  if (st) return st;
  if (N < 0 || C < 0 || HW < 0) return fail(OX_ERR_SHAPE, "%s: negative size (N=%lld C=%lld HW=%lld)", fn,
                                            (long long)N, (long long)C, (long long)HW);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(OX_ERR_INVALID_ARG, "%s: eps=%g is not a positive finite value", fn, (double)eps);
  const int64_t total = N * C * HW;
  if (C > INT32_MAX || HW > INT32_MAX || (HW > 0 && C > 0 && N > INT64_MAX / C / HW))
    return fail(OX_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (total > 0) {
    if (!X || !Y) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is NULL", fn);
    if (!gamma || !beta || !mean || !var) return fail(OX_ERR_INVALID_ARG, "%s: a BatchNorm parameter is NULL", fn);
    const size_t es = t == OX_F32 ? 4 : 2;
    if ((uintptr_t)X % es || (uintptr_t)Y % es) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is misaligned", fn);
  }
  if (total == 0) return ok();
  PoolArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = (int)t;
  a.total = total;
  a.planes = N * C;
  a.C = (int)C;
  a.HW = (int)HW;
  a.X = X;
  a.Y = Y;
  a.gamma = gamma;
  a.beta = beta;
  a.mean = mean;
  a.var = var;
  a.eps = eps;
  a.act = (int)act;
  return hip_result(fn, launch_bn_act(a, stream));
}

ox_status ox_maxpool2d(ox_dtype t, const ox_conv_desc* d, const void* X, void* Y, void* stream) {
  const char* fn = "ox_maxpool2d";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  if (!d) return fail(OX_ERR_INVALID_ARG, "%s: d is NULL", fn);
  if (d->M != d->C || d->group != 1)
    return fail(OX_ERR_INVALID_ARG, "%s: a pooling descriptor needs M == C and group == 1", fn);
  int64_t Ho, Wo;
  st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  // every window must reach the image (ONNX: pads smaller than the kernel extent)
  const int64_t eh = (d->kH - 1) * d->d_h + 1, ew = (d->kW - 1) * d->d_w + 1;
  if (d->p_t >= eh || d->p_b >= eh || d->p_l >= ew || d->p_r >= ew)
    return fail(OX_ERR_INVALID_ARG, "%s: a pad reaches the kernel extent (a window of padding only)", fn);
  const int64_t outs = d->N * d->C * Ho * Wo;
  if (outs > 0) {
    if (!X || !Y) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is NULL", fn);
    const size_t es = t == OX_F32 ? 4 : 2;
    if ((uintptr_t)X % es || (uintptr_t)Y % es) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is misaligned", fn);
  } else {
    return ok();
  }
  // the depthwise kernel's staged band, where its LDS band fits; else one
  // thread per output (OX_POOL_SIMPLE=1 forces the latter, for tests)
  const char* simple = getenv("OX_POOL_SIMPLE");
  if (!(simple && simple[0] == '1')) {
    ox_conv_desc dd = *d;
    dd.group = d->C;
    ConvArgs ca = conv_args((int)t, &dd, Ho, Wo, X, nullptr, nullptr, Y, ACT_NONE);
    if (depthwise_fits(ca)) return hip_result(fn, launch_maxpool_dw(ca, stream));
  }
  PoolArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = (int)t;
  a.planes = d->N * d->C;
  a.H = (int)d->H;
  a.W = (int)d->W;
  a.Ho = (int)Ho;
  a.Wo = (int)Wo;
  a.kH = (int)d->kH;
  a.kW = (int)d->kW;
  a.sh = (int)d->s_h;
  a.sw = (int)d->s_w;
  a.pt = (int)d->p_t;
  a.pl = (int)d->p_l;
  a.dh = (int)d->d_h;
  a.dw = (int)d->d_w;
  a.X = X;
  a.Y = Y;
  return hip_result(fn, launch_maxpool(a, stream));
}

ox_status ox_global_avgpool(ox_dtype t, int64_t N, int64_t C, int64_t HW, const void* X, void* Y,
                            void* stream) {
  const char* fn = "ox_global_avgpool";
  ox_status st = check_float_dt(fn, t);
  if (st) return st;
  if (N < 0 || C < 0 || HW < 1)
    return fail(OX_ERR_SHAPE, "%s: N=%lld C=%lld HW=%lld (HW must be at least 1)", fn, (long long)N,
                (long long)C, (long long)HW);
  if (HW > INT32_MAX || (C > 0 && N > INT64_MAX / C / HW))
    return fail(OX_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (N * C == 0) return ok();
  if (!X || !Y) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is NULL", fn);
  const size_t es = t == OX_F32 ? 4 : 2;
  if ((uintptr_t)X % es || (uintptr_t)Y % es) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is misaligned", fn);
  PoolArgs a;
  memset(&a, 0, sizeof(a));
  a.dt = (int)t;
  a.planes = N * C;
  a.C = (int)std::min<int64_t>(C, INT32_MAX);
  a.HW = (int)HW;
  a.X = X;
  a.Y = Y;
  return hip_result(fn, launch_global_avgpool(a, stream));
}

ox_status ox_matmul_nbits(ox_dtype t, int64_t M, int64_t N, int64_t K, int bits, int block_size,
                          const void* A, const uint8_t* B, const float* scales,
                          const uint8_t* zero_points, const void* bias, void* Y, void* stream) {
  const char* fn = "ox_matmul_nbits";
  if (t != OX_BF16) return fail(OX_ERR_UNSUPPORTED, "%s: dtype %d is not OX_BF16", fn, (int)t);
  if (bits != 4 || block_size != 32)
    return fail(OX_ERR_UNSUPPORTED, "%s: bits=%d block_size=%d (only 4-bit blocks of 32)", fn, bits,
                block_size);
  if (M < 0 || N < 0 || K < 0)
    return fail(OX_ERR_SHAPE, "%s: negative size M=%lld N=%lld K=%lld", fn, (long long)M,
                (long long)N, (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX - 64)
    return fail(OX_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (M * N == 0) return ok();
  if (!Y) return fail(OX_ERR_INVALID_ARG, "%s: Y is NULL", fn);
  if (K > 0 && (!A || !B || !scales)) return fail(OX_ERR_INVALID_ARG, "%s: A, B or scales is NULL", fn);
  if ((uintptr_t)A % 2 || (uintptr_t)Y % 2 || (uintptr_t)bias % 2 || (uintptr_t)B % 4 ||
      (uintptr_t)scales % 4)
    return fail(OX_ERR_INVALID_ARG, "%s: A / Y / bias must be 2-byte and B / scales 4-byte aligned", fn);
  NBitsArgs a;
  memset(&a, 0, sizeof(a));
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.nblk = (int)((K + 31) / 32);
  a.A = A;
  a.lda = K;
  a.a_vec = ((uintptr_t)A % 16) == 0 && K % 8 == 0;
  a.B = B;
  a.scales = scales;
  a.zp = zero_points;
  a.bias = bias;
  a.Y = Y;
  a.ldy = N;
  return hip_result(fn, launch_matmul_nbits(a, stream));
}

size_t ox_dynamic_quantize_workspace_bytes(void) { return dynq_workspace_bytes(); }

ox_status ox_dynamic_quantize_linear(int64_t n, const float* X, uint8_t* Y, float* y_scale,
                                     uint8_t* y_zp, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const char* fn = "ox_dynamic_quantize_linear";
  if (n < 0) return fail(OX_ERR_SHAPE, "%s: n=%lld is negative", fn, (long long)n);
  if (!y_scale || !y_zp) return fail(OX_ERR_INVALID_ARG, "%s: y_scale or y_zp is NULL", fn);
  if (n > 0 && (!X || !Y)) return fail(OX_ERR_INVALID_ARG, "%s: X or Y is NULL", fn);
  if ((uintptr_t)X % 4 || (uintptr_t)y_scale % 4)
    return fail(OX_ERR_INVALID_ARG, "%s: X or y_scale is not 4-byte aligned", fn);
  if (!workspace || workspace_bytes < dynq_workspace_bytes() || (uintptr_t)workspace % 16)
    return fail(OX_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned and hold %zu bytes", fn,
                dynq_workspace_bytes());
  return hip_result(fn, launch_dynamic_quantize(n, X, Y, y_scale, y_zp, workspace, stream));
}

ox_status ox_conv2d_variant(ox_dtype t, const ox_conv_desc* d, char* name, size_t cap) {
  const char* fn = "ox_conv2d_variant";
  if (t != OX_F32 && t != OX_BF16 && t != OX_I8)
    return fail(OX_ERR_UNSUPPORTED, "%s: dtype %d is not OX_F32, OX_BF16 or OX_I8", fn, (int)t);
  if (!name || cap == 0) return fail(OX_ERR_INVALID_ARG, "%s: name is NULL or cap is 0", fn);
  int64_t Ho, Wo;
  ox_status st = check_conv_desc(fn, d, &Ho, &Wo);
  if (st) return st;
  ConvArgs a = conv_args((int)t, d, Ho, Wo, nullptr, nullptr, nullptr, nullptr, ACT_NONE);
  const Force f = read_force();
  int kind;
  st = select_conv(fn, d, a, f, &kind);
  if (st) return st;
  int tile = -1;
  if (kind == KIND_IGEMM || kind == KIND_1X1) {
    st = pick_tile(fn, f, d->M / d->group, d->N * Ho * Wo, d->group, &tile,
                   t != OX_F32 ? RULE_CONV : kind == KIND_IGEMM ? RULE_IGEMM_F32
                   : d->C / d->group >= 64 ? RULE_1X1_F32 : RULE_CONV);
    if (st) return st;
  }
  static const char* dtn[] = {"f32", "bf16", "i8"};
  snprintf(name, cap, "%s/%s%s%s", kind_name(kind),
           dtn[(int)t], tile >= 0 ? "/" : "", tile >= 0 ? tile_name(tile) : "");
  return ok();
}

ox_status ox_fold_batchnorm(int64_t M, int64_t Kper, const float* W, const float* b0,
                            const float* gamma, const float* beta, const float* mean,
                            const float* var, float eps, float* W_out, float* b_out) {
  const char* fn = "ox_fold_batchnorm";
  if (M < 0 || Kper < 0) return fail(OX_ERR_INVALID_ARG, "%s: negative size", fn);
  if (M == 0) return ok();
  if (!gamma || !beta || !mean || !var || !b_out)
    return fail(OX_ERR_INVALID_ARG, "%s: gamma, beta, mean, var and b_out must not be NULL", fn);
  if (Kper > 0 && (!W || !W_out)) return fail(OX_ERR_INVALID_ARG, "%s: W or W_out is NULL", fn);
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(OX_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  for (int64_t m = 0; m < M; ++m) {
    const double den = (double)var[m] + (double)eps;
    if (!(den > 0.0))
      return fail(OX_ERR_INVALID_ARG, "%s: var[%lld] + eps = %g is not > 0", fn, (long long)m, den);
  }
  for (int64_t m = 0; m < M; ++m) {
    const double scale = (double)gamma[m] / sqrt((double)var[m] + (double)eps);
    const double shift = (double)beta[m] - (double)mean[m] * scale;
    for (int64_t k = 0; k < Kper; ++k) W_out[m * Kper + k] = (float)(scale * (double)W[m * Kper + k]);
    b_out[m] = (float)(scale * (b0 ? (double)b0[m] : 0.0) + shift);
  }
  return ok();
}

size_t ox_int8_params_bytes(int64_t M) {
  if (M < 0) return 0;
  return sizeof(Int8Header) + (size_t)M * (sizeof(double) + 2 * sizeof(int32_t));
}

ox_status ox_int8_prepare_ex(int64_t M, int64_t Kper, const int8_t* Wq_host, const int32_t* w_zp,
                             const float* w_scale, float x_scale, int32_t x_zp, int x_unsigned,
                             float y_scale, int32_t y_zp, int y_unsigned, const int32_t* bias_q,
                             void* params_host_out) {
  const char* fn = "ox_int8_prepare";
  if (M < 0 || Kper < 0) return fail(OX_ERR_INVALID_ARG, "%s: negative size", fn);
  if (!params_host_out) return fail(OX_ERR_INVALID_ARG, "%s: params_host_out is NULL", fn);
  if (M > 0 && !w_scale) return fail(OX_ERR_INVALID_ARG, "%s: w_scale is NULL", fn);
  if (M > 0 && Kper > 0 && !Wq_host) return fail(OX_ERR_INVALID_ARG, "%s: Wq_host is NULL", fn);
  const int32_t xlo = x_unsigned ? 0 : -128, ylo = y_unsigned ? 0 : -128;
  if (x_zp < xlo || x_zp > xlo + 255)
    return fail(OX_ERR_INVALID_ARG, "%s: x_zp=%d outside [%d,%d]", fn, x_zp, xlo, xlo + 255);
  if (y_zp < ylo || y_zp > ylo + 255)
    return fail(OX_ERR_INVALID_ARG, "%s: y_zp=%d outside [%d,%d]", fn, y_zp, ylo, ylo + 255);
  if (!(x_scale > 0.0f) || !isfinite(x_scale)) return fail(OX_ERR_INVALID_ARG, "%s: x_scale must be finite and > 0", fn);
  if (!(y_scale > 0.0f) || !isfinite(y_scale)) return fail(OX_ERR_INVALID_ARG, "%s: y_scale must be finite and > 0", fn);
  bool any_wzp = false;
  for (int64_t m = 0; m < M; ++m) {
    if (!(w_scale[m] > 0.0f) || !isfinite(w_scale[m]))
      return fail(OX_ERR_INVALID_ARG, "%s: w_scale[%lld] must be finite and > 0", fn, (long long)m);
    if (w_zp && (w_zp[m] < -128 || w_zp[m] > 127))
      return fail(OX_ERR_INVALID_ARG, "%s: w_zp[%lld]=%d outside [-128,127]", fn, (long long)m, w_zp[m]);
    if (w_zp && w_zp[m] != 0) any_wzp = true;
  }
  // the kernels read a uint8 tensor as int8 with the top bit flipped (u - 128)
  const int32_t xz = x_unsigned ? x_zp - 128 : x_zp;
  // Exact int32 range check, per output channel, over every activation the
  // type allows (int8 view x in [-128, 127], so x - x_zp in [-lo, hi]):
  //  * the true accumulator sum (x - x_zp)(w - w_zp[m]) + bias_q[m] lies in
  //    [bias - (lo*P + hi*Q), bias + (hi*P + lo*Q)], with P and Q the sums of
  //    the positive parts and of the magnitudes of the negative parts of
  //    w - w_zp[m];
  //  * the kernels' raw int8 x int8 sums (sum x*w, before the folded bias)
  //    lie in [-(128*Pw + 127*Qw), 127*Pw + 128*Qw] for the raw weights.
  // A channel whose range leaves int32 for some input is refused.
  {
    const int64_t lo = (int64_t)xz + 128, hi = 127 - (int64_t)xz;
    const int64_t imax = INT32_MAX, imin = INT32_MIN;
    for (int64_t m = 0; m < M; ++m) {
      const int64_t z = w_zp ? w_zp[m] : 0;
      int64_t P = 0, Q = 0, Pw = 0, Qw = 0;
      for (int64_t k = 0; k < Kper; ++k) {
        const int64_t w = Wq_host[m * Kper + k], d = w - z;
        if (d > 0) P += d; else Q -= d;
        if (w > 0) Pw += w; else Qw -= w;
      }
      const int64_t b = bias_q ? (int64_t)bias_q[m] : 0;
      if (b + hi * P + lo * Q > imax || b - (lo * P + hi * Q) < imin ||
          127 * Pw + 128 * Qw > imax || -(128 * Pw + 127 * Qw) < imin)
        return fail(OX_ERR_UNSUPPORTED,
                    "%s: channel %lld (Kper=%lld) could overflow the int32 accumulator for some input",
                    fn, (long long)m, (long long)Kper);
    }
  }
  const int32_t yz = y_unsigned ? y_zp - 128 : y_zp;
  char* out = (char*)params_host_out;
  Int8Header h;
  memset(&h, 0, sizeof(h));
  h.magic = kInt8Magic;
  h.version = 2;
  h.M = M;
  h.x_zp = xz;
  h.y_zp = yz;
  h.flags = (x_unsigned ? kI8XUnsigned : 0) | (y_unsigned ? kI8YUnsigned : 0) | (any_wzp ? kI8WZp : 0);
  memcpy(out, &h, sizeof(h));
  double* mult = (double*)(out + sizeof(Int8Header));
  int32_t* bfold = (int32_t*)(out + sizeof(Int8Header) + 8 * M);
  int32_t* wz = bfold + M;
  for (int64_t m = 0; m < M; ++m) {
    int64_t wsum = 0;
    for (int64_t k = 0; k < Kper; ++k) wsum += Wq_host[m * Kper + k];
    // sum (x - x_zp) w = sum x w - x_zp sum w, in the int8 view
    const int64_t bf = (bias_q ? (int64_t)bias_q[m] : 0) - (int64_t)xz * wsum;
    if (bf >= ((int64_t)1 << 31) || bf < -((int64_t)1 << 31))
      return fail(OX_ERR_UNSUPPORTED, "%s: folded bias of channel %lld overflows int32", fn, (long long)m);
    const double mm = ((double)x_scale * (double)w_scale[m]) / (double)y_scale;
    memcpy(mult + m, &mm, sizeof(double));
    const int32_t b32 = (int32_t)bf;
    memcpy(bfold + m, &b32, sizeof(int32_t));
    const int32_t z32 = w_zp ? w_zp[m] : 0;
    memcpy(wz + m, &z32, sizeof(int32_t));
  }
  return ok();
}

ox_status ox_int8_prepare(int64_t M, int64_t Kper, const int8_t* Wq_host, const float* w_scale,
                          float x_scale, int32_t x_zp, float y_scale, int32_t y_zp,
                          const int32_t* bias_q, void* params_host_out) {
  return ox_int8_prepare_ex(M, Kper, Wq_host, nullptr, w_scale, x_scale, x_zp, 0, y_scale, y_zp, 0,
                            bias_q, params_host_out);
}

}  // extern "C"
