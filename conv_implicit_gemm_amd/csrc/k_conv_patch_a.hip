// k_conv_patch_a.hip -- 64-channel configurations of the LDS-patch 3x3 kernel
// (one wave row of four waves, 64 or 32 pixels per wave).
#include "conv_patch.hpp"

namespace ox {

int launch_patch_1_4_2(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<1, 4, 2>(a, p, (hipStream_t)s);
}

int launch_patch_1_4_1(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<1, 4, 1>(a, p, (hipStream_t)s);
}

}  // namespace ox
