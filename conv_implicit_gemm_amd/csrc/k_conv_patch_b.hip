// k_conv_patch_b.hip -- 128-channel configurations of the LDS-patch 3x3
// kernel (2 x 2 waves, 64 or 32 pixels per wave).
#include "conv_patch.hpp"

namespace ox {

int launch_patch_2_2_2(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<2, 2, 2>(a, p, (hipStream_t)s);
}

int launch_patch_2_2_1(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<2, 2, 1>(a, p, (hipStream_t)s);
}

}  // namespace ox
