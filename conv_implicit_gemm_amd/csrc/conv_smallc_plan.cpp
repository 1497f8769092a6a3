// conv_smallc_plan.cpp -- host-side planning of the few-input-channel kernel.
#include <algorithm>
#include <cstdlib>
#include <cstdint>
#include <cstdio>

#include "ox_internal.h"

namespace ox {

int launch_smallc(const ConvArgs& a, const SmallcPlan& p, void* stream);

namespace {

constexpr int kLdsMax = 160 * 1024;

bool geometry(const ConvArgs& a) {
  return a.dt == DT_BF16 && a.group == 1 && a.C >= 1 && a.C <= 4 && a.dh == 1 && a.dw == 1 &&
         a.sh == a.sw && (a.sh == 1 || a.sh == 2) && a.kW >= 1 && a.kW <= 8 && a.kH >= 1 &&
         a.kH <= 16;
}

bool make(const ConvArgs& a, int FP, SmallcPlan* out) {
  SmallcPlan p;
  p.FP = FP;
  p.NH = a.kW <= 4 ? 1 : 2;
  p.P = (a.W % 8 == 0 && ((uintptr_t)a.X) % 16 == 0) ? 8 : 1;
  const int slots = 4 * FP * 32;
  if (a.Wo > slots) return false;
  const int trmax = std::min(a.Ho, slots / a.Wo);
  p.nrb = (a.Ho + trmax - 1) / trmax;
  p.TR = (a.Ho + p.nrb - 1) / p.nrb;
  p.PR = (p.TR - 1) * a.sh + a.kH;
  p.PWc = a.sw * (a.Wo - 1) + 4 * p.NH;
  p.PWc += p.PWc & 1;
  p.nmb = (a.M + 63) / 64;
  const int wrow = a.kH * p.NH * 32 + 16;
  const int wraw = ((64 * a.C * a.kH * a.kW * 2) + 15) / 16 * 16;   // weight rows as stored
  p.lds = std::max(64 * wrow + p.PR * p.PWc * 8 + wraw, 64 * (slots + 8) * 2);
  p.w_vec = ((uintptr_t)a.Wt) % 16 == 0;   // a block's rows start 128*K bytes apart
  if (p.lds > kLdsMax || (int64_t)p.nrb * a.N * p.nmb >= ((int64_t)1 << 31)) return false;
  *out = p;
  return true;
}

// 512-pixel blocks (four tiles per wave) where a row fits and the grid
// still has two blocks per CU; else 256-pixel blocks
bool plan(const ConvArgs& a, SmallcPlan* out) {
  if (!geometry(a)) return false;
  if (const char* e = getenv("OX_SMALLC_FP")) {   // pins the tiles per wave (measurements)
    const int fp = atoi(e) == 2 ? 2 : 4;
    return make(a, fp, out);
  }
  SmallcPlan p4;
  if (make(a, 4, &p4) && (int64_t)p4.nrb * a.N * p4.nmb >= 512) {
    *out = p4;
    return true;
  }
  return make(a, 2, out) || make(a, 4, out);
}

}  // namespace

bool conv_smallc_applicable(const ConvArgs& a) {
  SmallcPlan p;
  return plan(a, &p);
}

int launch_conv_smallc(const ConvArgs& a, void* stream) {
  SmallcPlan p;
  if (!plan(a, &p)) return 1;   // hipErrorInvalidValue
  return launch_smallc(a, p, stream);
}

const char* conv_smallc_describe(const ConvArgs& a, char* buf, int cap) {
  SmallcPlan p;
  if (!plan(a, &p)) return "";
  snprintf(buf, cap, "FP=%d NH=%d P=%d TR=%d PR=%d PWc=%d blocks=%lld lds=%d wvec=%d", p.FP, p.NH, p.P,
           p.TR, p.PR, p.PWc, (long long)p.nrb * a.N * p.nmb, p.lds, p.w_vec);
  return buf;
}

}  // namespace ox
