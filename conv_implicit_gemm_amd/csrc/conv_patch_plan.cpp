// conv_patch_plan.cpp -- host-side planning of the LDS-patch 3x3 kernel:
// which configuration (wave grid, pixel tiles per wave) and which band of
// output rows / images each block owns.  Pure host code.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ox_internal.h"

namespace ox {

int launch_patch_1_4_2(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_1_4_1(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_2_2_2(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_2_2_1(const ConvArgs& a, const PatchPlan& p, void* s);

namespace {

constexpr int kCell = 80;
constexpr int kLdsMax = 160 * 1024;
constexpr int kCUs = 256;

// wave grid WM x (4/WM), FP 32-pixel tiles per wave, two 32-channel tiles
// per wave: a block covers 64*WM channels and 32*(4/WM)*FP pixel slots
struct Cfg {
  int WM, FP;
};
const Cfg kCfgs[] = {{1, 2}, {1, 1}, {2, 2}, {2, 1}};

int slots_of(const Cfg& c) { return 32 * (4 / c.WM) * c.FP; }

PatchPlan make(const ConvArgs& a, const Cfg& c, int TR, int IMB) {
  PatchPlan p;
  p.BM = 64 * c.WM;
  p.WM = c.WM;
  p.FN = c.FP;
  p.TR = TR;
  p.IMB = IMB;
  p.PR = (TR - 1) * a.sh + 2 * a.dh + 1;
  p.PW = (a.Wo - 1) * a.sw + 2 * a.dw + 1;
  p.PWs = (p.PW + a.sw - 1) / a.sw;
  p.PWt = p.PWs * a.sw;
  p.NT = (IMB * TR * a.Wo + 31) / 32;
  p.nrb = (a.Ho + TR - 1) / TR;
  p.nib = (a.N + IMB - 1) / IMB;
  p.nmb = (a.M + p.BM - 1) / p.BM;
  p.npos = IMB * p.PR * p.PWt;
  const int HW = a.H * a.W;
  // positions per staging unit (P): the widest load (P bf16) that every
  // plane's start keeps aligned
  p.VW = (HW % 8 == 0) ? 8 : (HW % 4 == 0) ? 4 : (HW % 2 == 0) ? 2 : 1;
  {
    // staging units per thread (the kernel's patch_upt): 64 (P = 1) or 32
    // staging registers, halved for 128-channel blocks, at least one unit
    const int dwords = p.VW <= 2 ? 8 : 4 * p.VW;
    const int upt = (p.VW == 1 ? 64 : 32) / (p.BM >= 128 ? 2 : 1) / dwords;
    p.UPT = upt > 0 ? upt : 1;
  }
  // staging units: images x 4 channel octets x groups of P plane positions
  // (a band of R rows spans at most R*W + P - 1 positions from a P-aligned start)
  const int rows = std::min(a.H, p.PR);
  p.units = IMB * 4 * ((rows * a.W + 2 * p.VW - 2) / p.VW);
  p.lds = p.BM * (9 * 64 + 16) + p.npos * kCell   // weight rows and patch cells
          + p.BM * 4;                             // + the tile's fp32 bias
  p.splits = 1;
  p.cps = std::max(1, a.C / 32);
  p.ws = nullptr;
  p.ga = p.gb = 1;
  return p;
}

// XCD rectangles (see tile_geo): each of the 8 XCDs takes (pixel blocks /
// ga) x (channel blocks / gb) tiles, so every input band is fetched into gb
// L2s and every weight row into ga.  Pick the split of 8 = ga*gb (exact
// divisions only) with the fewest estimated L2 fill bytes, against the plain
// channel-block-major order (bands into ~nmb L2s, weights into ~8/nmb).
void set_groups(const ConvArgs& a, PatchPlan* p) {
  p->ga = p->gb = 1;
  const int npb = p->nrb * p->nib;
  const double xb = (double)a.N * a.C * a.H * a.W * 2, wb = (double)a.M * a.C * 9 * 2;
  const int nm = p->nmb;
  double best = xb * std::min(nm, 8) + wb * std::max(1.0, 8.0 / nm);
  if (const char* e = getenv("OX_PATCH_XCD")) {
    int ga, gb;
    if (sscanf(e, "%d:%d", &ga, &gb) == 2 && ga * gb == 8 && npb % ga == 0 && nm % gb == 0) {
      p->ga = ga;
      p->gb = gb;
    }
    return;
  }
  for (int gb = 1; gb <= 8; gb *= 2) {
    const int ga = 8 / gb;
    if (npb % ga || nm % gb) continue;
    const double c = xb * gb + wb * ga;
    if (c < best * 0.97) {
      best = c;
      p->ga = ga;
      p->gb = gb;
    }
  }
}

// split the channel chunks of each tile into `splits` slices (at least one chunk each)
void set_splits(const ConvArgs& a, PatchPlan* p, int splits) {
  const int nchunks = std::max(1, a.C / 32);
  splits = std::max(1, std::min(splits, nchunks));
  p->cps = (nchunks + splits - 1) / splits;
  p->splits = (nchunks + p->cps - 1) / p->cps;
}

size_t ws_bytes(const PatchPlan& p) {
  const int FP = p.FN;
  return p.splits > 1 ? (size_t)p.nrb * p.nib * p.nmb * p.splits * 8192 * FP * sizeof(float) : 0;
}

bool fits(const PatchPlan& p) {
  const int ntmax = (4 / p.WM) * p.FN;
  return p.NT <= ntmax && p.lds <= kLdsMax && p.units <= p.UPT * 256 &&
         (int64_t)p.nrb * p.nib * p.nmb * p.splits < (1 << 22);
}

// Rough time model: MFMA cycles per SIMD over the whole grid against the
// bytes the blocks pull through L2 (every pixel block reads all weights of its
// channel block; every channel block re-reads the input band with its halo).
double cost(const ConvArgs& a, const PatchPlan& p) {
  const double mblocks = (a.M + p.BM - 1) / p.BM;
  const double pblocks = (double)p.nrb * p.nib;
  const double blocks = mblocks * pblocks;
  const int per_cu = std::max(1, std::min(p.BM == 64 ? 2 : 1, kLdsMax / p.lds));
  // per wave and chunk: 18 k-steps x FP x 2 MFMAs of 32 cycles
  const double waves_cycles = (a.C / 32) * 18.0 * p.FN * 2 * 32.0;
  const double rounds = std::ceil(blocks / (kCUs * per_cu));
  const double t_mfma = rounds * per_cu * waves_cycles / 2.4e9;
  const double wbytes = (double)a.M * a.C * 9 * 2;
  const double xbytes = (double)a.N * a.C * a.H * a.W * 2;
  const double halo = (double)std::min(a.H, p.PR) / std::max(1.0, (double)p.TR * a.sh);
  const double traffic = wbytes * pblocks + xbytes * mblocks * std::max(1.0, halo);
  const double t_mem = traffic / 6e12;
  // per-chunk fixed cost (two barriers and an exposed load latency), per round
  const double t_fix = rounds * (a.C / 32) * 0.25e-6;
  return std::max(t_mfma, t_mem) + t_fix;
}

// the tallest band of at most `slots` pixels, evened out over the image so
// that the last band is not a sliver -- or, among the heights that give the
// same number of bands, one whose bands start at a multiple of four output
// pixels (8-byte aligned bf16 rows: the epilogue stores four pixels at once
// only there; 14x14 layers, 8-row bands instead of 7: ~10% faster)
int band_rows(const ConvArgs& a, int slots) {
  const int trmax = std::max(1, std::min(a.Ho, slots / std::max(1, a.Wo)));
  const int nrb = (a.Ho + trmax - 1) / trmax;
  const int even = (a.Ho + nrb - 1) / nrb;
  if ((even * a.Wo) % 4 == 0 || nrb == 1) return even;
  for (int tr = trmax; tr > even; --tr)
    if ((tr * a.Wo) % 4 == 0 && (a.Ho + tr - 1) / tr == nrb) return tr;
  return even;
}

}  // namespace

// OX_PATCH_PLAN=WM:FP:TR:IMB[:S] pins the plan (for measurements), S being
// the split-K slice count (taken only when the call brings a workspace); a
// pinned plan that does not fit this geometry makes the kernel inapplicable.
bool pinned_plan(const ConvArgs& a, PatchPlan* out, bool* pinned) {
  const char* e = getenv("OX_PATCH_PLAN");
  *pinned = false;
  if (!e || !*e) return false;
  int wm, fp, tr, imb, sk = 1;
  if (sscanf(e, "%d:%d:%d:%d:%d", &wm, &fp, &tr, &imb, &sk) < 4) return false;
  *pinned = true;
  for (const Cfg& c : kCfgs) {
    if (c.WM != wm || c.FP != fp) continue;
    if (tr < 1 || tr > a.Ho || imb < 1 || (imb > 1 && tr != a.Ho)) return false;
    PatchPlan p = make(a, c, tr, imb);
    set_splits(a, &p, a.ws ? sk : 1);
    if (!fits(p)) return false;
    set_groups(a, &p);
    *out = p;
    return true;
  }
  return false;
}

bool patch_plan(const ConvArgs& a, PatchPlan* out) {
  bool pinned;
  const bool ok = pinned_plan(a, out, &pinned);
  if (pinned) return ok;
  // Selection rule, from a sweep of every configuration, band height,
  // images per block and split count on the ResNet-50 3x3 layers at batch
  // 32 (MI355X): 64 output channels per block won on every shape; 128-pixel
  // blocks (one pixel tile per wave) won wherever such a block holds at least
  // three output rows, 256-pixel blocks on the wide 56-column layer.  The
  // band is the tallest that fits the block, evened out over the image.
  // Images of at most 64 output pixels go two or more to a block; when the
  // tiles then number fewer than 200, each tile's channel chunks are split
  // into slices of at least four chunks, up to ~512 work units (split-K:
  // two slices per CU-slot won on the 7x7 layers, where 16 chunks per tile
  // otherwise run back to back on half the CUs).
  {
    const int wo = std::max(1, a.Wo);
    const Cfg& c = (128 / wo >= 3 || a.Ho <= 128 / wo) ? kCfgs[1] : kCfgs[0];
    const int slots = slots_of(c);
    const int64_t img = (int64_t)a.Ho * a.Wo;
    bool got = false;
    PatchPlan p;
    if (img * 2 <= slots) {
      p = make(a, c, a.Ho, (int)(slots / img));
      got = fits(p);
    }
    for (int TR = band_rows(a, slots); !got && TR >= 1; --TR) {
      p = make(a, c, TR, 1);
      got = fits(p);
    }
    if (got) {
      const int64_t tiles = (int64_t)p.nrb * p.nib * p.nmb;
      const int nchunks = std::max(1, a.C / 32);
      if (a.ws && tiles < 200 && nchunks >= 8) {
        set_splits(a, &p, (int)std::min<int64_t>((512 + tiles - 1) / tiles, nchunks / 4));
        if (!fits(p)) set_splits(a, &p, 1);
      }
      set_groups(a, &p);
      *out = p;
      return true;
    }
  }
  bool found = false;
  double best = 1e30;
  // rows wider than a block: every configuration and band height
  for (const Cfg& c : kCfgs) {
    for (int TR = 1; TR <= a.Ho; ++TR) {
      const PatchPlan p = make(a, c, TR, 1);
      if (!fits(p)) continue;
      const double t = cost(a, p);
      if (t < best * 0.999) {
        best = t;
        *out = p;
        found = true;
      }
    }
  }
  return found;
}

bool conv_patch_geometry(const ConvArgs& a) {
  // operands are addressed with 32-bit buffer offsets (below 2^31 bytes);
  // the kernel's setup divisions need index ranges below 2^22
  return a.dt == DT_BF16 && a.group == 1 && a.kH == 3 && a.kW == 3 && a.C % 32 == 0 &&
         a.sh == a.sw && (a.sw == 1 || a.sw == 2) &&
         (int64_t)a.N * a.C * a.H * a.W * 2 < ((int64_t)1 << 31) &&
         (int64_t)a.M * a.C * 9 * 2 < ((int64_t)1 << 31) && (int64_t)a.H * a.W < (1 << 22);
}

bool conv_patch_applicable(const ConvArgs& a) {
  if (!conv_patch_geometry(a)) return false;
  if (!a.w_vec || (((uintptr_t)a.X) & 15) != 0) return false;
  PatchPlan p;
  return patch_plan(a, &p);
}

int launch_conv_patch(const ConvArgs& a, void* stream) {
  PatchPlan p;
  if (!patch_plan(a, &p)) return 1;  // hipErrorInvalidValue
  if (p.splits > 1) {
    if (!a.ws || a.ws_bytes < ws_bytes(p)) return 1;   // validated by the entry point
    p.ws = (float*)a.ws;
  }
  if (p.WM == 1) {
    return p.FN == 2 ? launch_patch_1_4_2(a, p, stream) : launch_patch_1_4_1(a, p, stream);
  }
  return p.FN == 2 ? launch_patch_2_2_2(a, p, stream) : launch_patch_2_2_1(a, p, stream);
}

size_t conv_patch_ws_bytes(const ConvArgs& a) {
  PatchPlan p;
  return patch_plan(a, &p) ? ws_bytes(p) : 0;
}

const char* conv_patch_describe(const ConvArgs& a, char* buf, int cap) {
  PatchPlan p;
  if (!patch_plan(a, &p)) return "";
  snprintf(buf, cap, "BM=%d WM=%d FP=%d TR=%d IMB=%d NT=%d VW=%d splits=%d xcd=%dx%d blocks=%lld lds=%d",
           p.BM, p.WM, p.FN, p.TR, p.IMB, p.NT, p.VW, p.splits, p.ga, p.gb,
           (long long)p.nrb * p.nib * p.nmb * p.splits, p.lds);
  return buf;
}

}  // namespace ox
