// k_conv_patch_a.hip -- 64-row configurations of the LDS-patch 3x3 kernel.
#include "conv_patch.hpp"

namespace ox {

int launch_patch_64_1_2(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<64, 1, 2>(a, p, (hipStream_t)s);
}

int launch_patch_64_1_4(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<64, 1, 4>(a, p, (hipStream_t)s);
}

}  // namespace ox
