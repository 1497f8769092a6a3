// conv_pw_plan.cpp -- host-side planning of the pointwise (1x1) kernel.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ox_internal.h"

namespace ox {

int launch_pw_1_32(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_1_64(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_2_32(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_2_64(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pwd_128_64_64(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_128_64_32(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_64_64_64(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_64_128_64(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_64_128_32(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_64_256_64(const ConvArgs& a, const PwdPlan& p, void* s);
int launch_pwd_64_256_32(const ConvArgs& a, const PwdPlan& p, void* s);

namespace {

constexpr int kLdsMax = 160 * 1024;
constexpr int kCUs = 256;        // kCUs is a multiple of the 8 XCDs
constexpr int kMaxPerCu = 3;

bool geometry(const ConvArgs& a) {
  return a.dt == DT_BF16 && a.group == 1 && a.kH == 1 && a.kW == 1 && a.sh == 1 && a.sw == 1 &&
         a.pt == 0 && a.pl == 0 && a.Ho == a.H && a.Wo == a.W && a.C % 32 == 0 && a.C > 0;
}

PwPlan make(const ConvArgs& a, int WM, int KC, int FP) {
  PwPlan p;
  p.WM = WM;
  p.FP = FP;
  p.KC = KC;
  const int HW = a.H * a.W;
  const uintptr_t xa = (uintptr_t)a.X, ya = (uintptr_t)a.Y;
  p.P = (HW % 4 == 0 && xa % 8 == 0) ? 4 : (HW % 2 == 0 && xa % 4 == 0) ? 2 : 1;
  const uintptr_t ra = (uintptr_t)a.res;     // residual (0: none), read in runs like Y
  p.V = 8;
  while (p.V > 1 && (HW % p.V || ya % (2 * p.V) || ra % (2 * p.V))) p.V >>= 1;
  const int BM = 64 * WM, BN = 32 * (4 / WM) * FP;
  const int64_t Q = (int64_t)a.N * HW;
  p.npb = (int)((Q + BN - 1) / BN);
  p.nmb = (a.M + BM - 1) / BM;
  const int row = KC * 2 + 16;
  // two operand buffers (or the epilogue's staging tile) + the bias vector
  // (raw bf16 words from its aligned-down address)
  p.bias_lds = ((2 * a.M + 3 + 3) / 4 * 4 + 15) / 16 * 16;
  p.lds = std::max(2 * (BM + BN) * row, BM * (BN + 8) * 2) + p.bias_lds;
  if (a.res) p.lds = std::max(p.lds, BM * (BN + 4) * 4 + p.bias_lds);   // fp32 staging of the residual epilogue
  // split-K when the tiles alone would leave many CUs idle and the channel
  // range is long: about 384 work units of at least four chunks (ResNet-50's
  // 2048->512 1x1 at 7x7, batch 32, 104 tiles x 32 chunks: 1 / 2 / 3 / 4
  // slices 34.1 / 22.4 / 21.9 / 20.2 us per call, the second pass storing
  // from registers)
  const int64_t tiles = (int64_t)p.npb * p.nmb;
  const int nchunks = std::max(1, a.C / KC);   // (a C that KC does not divide is rejected by valid)
  int target = 1;
  if (a.ws && tiles < 192 && nchunks >= 4)
    target = (int)std::min<int64_t>((384 + tiles - 1) / tiles, nchunks / 4);
  if (const char* e = getenv("OX_PW_SPLITS"))
    if (a.ws) target = std::max(1, std::min(nchunks, atoi(e)));
  p.cps = (nchunks + target - 1) / target;
  p.splits = (nchunks + p.cps - 1) / p.cps;
  p.ws = nullptr;
  // persistent grid: as many blocks as fit the chip at once (LDS-bound, at
  // most kMaxPerCu per CU), a multiple of the XCD count when units are left over
  int per_cu = std::max(1, std::min(kMaxPerCu, kLdsMax / p.lds));
  if (const char* e = getenv("OX_PW_PER_CU")) per_cu = std::max(1, std::min(kLdsMax / p.lds, atoi(e)));
  const int64_t units = tiles * p.splits;
  const int64_t cap = (int64_t)kCUs * per_cu;
  p.grid = (int)std::min(units, cap);
  // OX_PW_GRID=n pins the persistent grid (blocks then run several units
  // each: the path that crosses from one unit into the next)
  if (const char* e = getenv("OX_PW_GRID")) p.grid = (int)std::max<int64_t>(1, std::min<int64_t>(units, atoi(e)));
  return p;
}

size_t ws_bytes(const PwPlan& p) {
  const int BM = 64 * p.WM, BN = 32 * (4 / p.WM) * p.FP;
  return p.splits > 1 ? (size_t)p.npb * p.nmb * p.splits * BM * BN * sizeof(float) : 0;
}

bool valid(const ConvArgs& a, const PwPlan& p) {
  // (a block of two pixel fragments per wave staging single pixels takes
  // 32-channel chunks: the two register sets of 64 would spill)
  return a.C % p.KC == 0 && p.KC <= 64 && !(p.FP == 2 && p.P == 1 && p.KC > 32) &&
         p.lds <= kLdsMax && (int64_t)p.npb * p.nmb * p.splits < (int64_t)1 << 31 &&
         // byte offsets of the kernel's buffer loads are 32-bit
         (int64_t)a.N * a.C * a.H * a.W * 2 < (int64_t)1 << 30 && (int64_t)a.M * a.C * 2 < (int64_t)1 << 30 &&
         (int64_t)a.N * a.M * a.H * a.W < (int64_t)1 << 31;   // 32-bit element offsets into Y (and R)
}

// Pixel fragments per wave: two (128 x 128 or 64 x 256 tiles), or one where
// tiles of that size would leave CUs without a block -- half-width tiles
// double the block count, so that blocks share CUs and overlap one's staging
// with another's MFMAs (a sweep of the ResNet-50 1x1 layers at batch 32:
// -28% at 208 tiles, -12% at 98, -3% at 196, but +8..+26% at 392).
// OX_PW_FP pins it.
int fp_choice(const ConvArgs& a, int WM) {
  if (const char* e = getenv("OX_PW_FP")) return atoi(e) == 1 ? 1 : 2;
  const int64_t Q = (int64_t)a.N * a.H * a.W;
  const int BM = 64 * WM, BN = 32 * (4 / WM) * 2;
  const int64_t tiles = ((Q + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  return tiles < kCUs ? 1 : 2;
}

// OX_PW_PLAN=WM:KC pins the configuration (for measurements); a pinned
// configuration that does not apply makes the kernel inapplicable.
bool pw_plan(const ConvArgs& a, PwPlan* out) {
  if (!geometry(a)) return false;
  const char* e = getenv("OX_PW_PLAN");
  int wm, kc;
  if (e && *e && sscanf(e, "%d:%d", &wm, &kc) == 2) {
    if ((wm != 1 && wm != 2) || (kc != 32 && kc != 64)) return false;
    const PwPlan p = make(a, wm, kc, fp_choice(a, wm));
    if (!valid(a, p)) return false;
    *out = p;
    return true;
  }
  // 64-channel blocks when M fits one, else 128 x 128.  Chunks of 64
  // channels (fewer barriers, more bytes in flight per chunk) unless that
  // leaves a single chunk per tile (nothing for the second operand buffer to
  // overlap) or does not fit two blocks per CU; then 32 (a sweep of the
  // ResNet-50 1x1 layers at batch 32: -28% for C = 256 at 64 x 256 tiles,
  // -17% for C = 64)
  const int WM = a.M <= 64 ? 1 : 2;
  const int FP = fp_choice(a, WM);
  const PwPlan p64 = make(a, WM, 64, FP);
  if (valid(a, p64) && a.C / 64 >= 2 && 2 * p64.lds <= kLdsMax) {
    *out = p64;
    return true;
  }
  const PwPlan p32 = make(a, WM, 32, FP);
  if (valid(a, p32)) {
    *out = p32;
    return true;
  }
  if (valid(a, p64)) {
    *out = p64;
    return true;
  }
  return false;
}

// ---------------------------------------------------- DMA-staged kernel --
//
// Configurations (BP pixels x BC channels, KC channels per stage, S stages,
// WP waves along the pixels) -- each one instantiation in k_conv_pwd.hip:
struct PwdCfg {
  int BP, BC, KC, S, WP;
  int (*launch)(const ConvArgs&, const PwdPlan&, void*);
};
const PwdCfg kPwdCfgs[] = {
    {128, 64, 64, 3, 4, launch_pwd_128_64_64}, {128, 64, 32, 4, 4, launch_pwd_128_64_32},
    {64, 64, 64, 4, 2, launch_pwd_64_64_64},
    {64, 128, 64, 3, 2, launch_pwd_64_128_64}, {64, 128, 32, 4, 2, launch_pwd_64_128_32},
    {64, 256, 64, 2, 1, launch_pwd_64_256_64}, {64, 256, 32, 3, 1, launch_pwd_64_256_32},
};

int pwd_lds(const PwdCfg& c, bool res) {
  const int slot = c.KC * c.BP * 2 + c.BC * c.KC * 2, stage = c.BC * (c.BP * 2 + 8);
  return c.S * slot + (res || stage <= slot ? 0 : stage);
}

bool aligned_to(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

const PwdCfg* find_cfg(int BP, int BC, int KC) {
  for (const PwdCfg& c : kPwdCfgs)
    if (c.BP == BP && c.BC == BC && c.KC == KC) return &c;
  return nullptr;
}

// Blocks of the persistent grid for a configuration (ranges of 64 or 128
// pixels x channel blocks), and the range split: pixel ranges are k whole
// units of 128 pixels -- 64 where 128 would leave fewer than 256 blocks --
// with k the least that fits the grid (at most as many blocks as fit the
// chip at once), so that every block gets the same work.  OX_PWD_GRID caps
// the block count (a test of ranges with several tiles).
void split_ranges(const ConvArgs& a, int64_t Q, PwdPlan* p) {
  const int per_cu = std::max(1, std::min(2, kLdsMax / p->lds));
  int64_t cap = (int64_t)kCUs * per_cu;
  if (const char* g = getenv("OX_PWD_GRID")) cap = std::max(1, atoi(g));
  const int64_t units128 = (Q + 127) / 128;
  const int unit = units128 * p->nmb >= kCUs || cap < kCUs ? 128 : 64;
  const int64_t units = (Q + unit - 1) / unit;
  const int64_t per_range_cap = std::max<int64_t>(1, cap / p->nmb);
  const int64_t k = (units + per_range_cap - 1) / per_range_cap;
  p->span = (int)std::min<int64_t>(k * unit, (int64_t)1 << 30);
  p->nranges = (int)((units + k - 1) / k);
  p->grid = p->nranges * p->nmb;
  (void)a;
}

// The configuration for a shape.  Output channels per block: the largest of
// 256 / 128 / 64 (not beyond what M needs) that still gives 192 blocks --
// a wide block reads each pixel once, a narrow one gives small layers
// enough blocks without splitting K (ResNet-50's 1024->256 1x1 at 14x14,
// batch 32: 128 channels x 196 blocks 13.8 us against 64 x 392 16.7 us).  64-channel stages where C allows;
// 128-pixel tiles for 64-channel blocks when the pixels give 256 of them.
// Pixel pieces of 16 bytes when H*W % 8 == 0 (and X is 16-byte aligned),
// else 4 bytes when H*W is even.  OX_PWD_CFG=BP:BC:KC pins a configuration.
bool pwd_plan(const ConvArgs& a, PwdPlan* out) {
  if (!geometry(a)) return false;
  const int64_t HW = (int64_t)a.H * a.W;
  const int64_t Q = (int64_t)a.N * HW;
  if (Q == 0 || !aligned_to(a.Wt, 16)) return false;
  int PB;
  if (HW % 8 == 0 && aligned_to(a.X, 16)) PB = 16;
  else if (HW % 2 == 0 && aligned_to(a.X, 4)) PB = 4;
  else return false;
  if (a.res && (PB != 16 || !aligned_to(a.Y, 16) || !aligned_to(a.res, 16))) return false;
  if ((int64_t)a.N * a.C * HW * 2 >= ((int64_t)1 << 30) || (int64_t)a.M * a.C * 2 >= ((int64_t)1 << 30) ||
      (int64_t)a.N * a.M * HW >= ((int64_t)1 << 31))
    return false;
  int V = 8;
  while (V > 1 && (HW % V || !aligned_to(a.Y, 2 * V))) V >>= 1;
  const int KC = a.C % 64 == 0 ? 64 : 32;
  const PwdCfg* cfg = nullptr;
  const char* e = getenv("OX_PWD_CFG");
  int BP = 0, BC = 0, KCp = 0;
  if (e && *e) {
    if (sscanf(e, "%d:%d:%d", &BP, &BC, &KCp) != 3) return false;
    cfg = find_cfg(BP, BC, KCp);
  } else {
    const int mcap = a.M <= 64 ? 64 : a.M <= 128 ? 128 : 256;
    for (int bc = mcap; bc >= 64 && !cfg; bc /= 2) {
      const PwdCfg* c = nullptr;
      if (bc == 64) {
        const bool wide = (Q + 127) / 128 * ((a.M + 63) / 64) >= kCUs;
        c = find_cfg(wide ? 128 : 64, 64, KC);
        if (!c) c = find_cfg(128, 64, KC);
      } else {
        c = find_cfg(64, bc, KC);
      }
      if (!c) continue;
      const int64_t nmb = (a.M + bc - 1) / bc;
      if ((Q + 63) / 64 * nmb >= kCUs * 3 / 4 || bc == 64) cfg = c;
    }
  }
  if (!cfg || a.C % cfg->KC != 0) return false;
  PwdPlan p;
  p.BP = cfg->BP;
  p.BC = cfg->BC;
  p.KC = cfg->KC;
  p.S = cfg->S;
  p.WP = cfg->WP;
  p.PB = PB;
  p.V = V;
  p.nmb = (a.M + p.BC - 1) / p.BC;
  p.Q = (int)Q;
  p.lds = pwd_lds(*cfg, a.res != nullptr);
  if (p.lds > kLdsMax) return false;
  split_ranges(a, Q, &p);
  if ((int64_t)p.nranges * p.nmb >= ((int64_t)1 << 31)) return false;
  p.hw = make_fastdiv((uint32_t)HW);
  p.x_bytes = (uint32_t)((int64_t)a.N * a.C * HW * 2);
  p.w_bytes = (uint32_t)((int64_t)a.M * a.C * 2);
  *out = p;
  return true;
}

const PwdCfg* pwd_cfg(const PwdPlan& p) {
  for (const PwdCfg& c : kPwdCfgs)
    if (c.BP == p.BP && c.BC == p.BC && c.KC == p.KC) return &c;
  return nullptr;
}

}  // namespace

bool conv_pwd_applicable(const ConvArgs& a) {
  PwdPlan p;
  return pwd_plan(a, &p);
}

int launch_conv_pwd(const ConvArgs& a, void* stream) {
  PwdPlan p;
  if (!pwd_plan(a, &p)) return 1;   // hipErrorInvalidValue
  return pwd_cfg(p)->launch(a, p, stream);
}

const char* conv_pwd_describe(const ConvArgs& a, char* buf, int cap) {
  PwdPlan p;
  if (!pwd_plan(a, &p)) return "";
  snprintf(buf, cap, "BP=%d BC=%d KC=%d S=%d WP=%d PB=%d V=%d ranges=%d span=%d grid=%d lds=%d", p.BP, p.BC,
           p.KC, p.S, p.WP, p.PB, p.V, p.nranges, p.span, p.grid, p.lds);
  return buf;
}

bool conv_pw_applicable(const ConvArgs& a) {
  if (!a.w_vec || ((uintptr_t)a.X) % 2 != 0) return false;
  PwPlan p;
  return pw_plan(a, &p);
}

int launch_conv_pw(const ConvArgs& a, void* stream) {
  PwPlan p;
  if (!pw_plan(a, &p)) return 1;   // hipErrorInvalidValue
  if (p.splits > 1) {
    if (!a.ws || a.ws_bytes < ws_bytes(p)) return 1;   // validated by the entry point
    p.ws = (float*)a.ws;
  }
  if (p.WM == 1) return p.KC == 64 ? launch_pw_1_64(a, p, stream) : launch_pw_1_32(a, p, stream);
  return p.KC == 64 ? launch_pw_2_64(a, p, stream) : launch_pw_2_32(a, p, stream);
}

size_t conv_pw_ws_bytes(const ConvArgs& a) {
  PwPlan p;
  return pw_plan(a, &p) ? ws_bytes(p) : 0;
}

const char* conv_pw_describe(const ConvArgs& a, char* buf, int cap) {
  PwPlan p;
  if (!pw_plan(a, &p)) return "";
  snprintf(buf, cap, "BM=%d BN=%d KC=%d P=%d V=%d tiles=%lld splits=%d grid=%d lds=%d", 64 * p.WM,
           32 * (4 / p.WM) * p.FP, p.KC, p.P, p.V, (long long)p.npb * p.nmb, p.splits, p.grid, p.lds);
  return buf;
}

}  // namespace ox
