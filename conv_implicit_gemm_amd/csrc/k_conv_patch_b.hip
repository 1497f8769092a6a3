// k_conv_patch_b.hip -- 128-row configurations of the LDS-patch 3x3 kernel.
#include "conv_patch.hpp"

namespace ox {

int launch_patch_128_2_7(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<128, 2, 7>(a, p, (hipStream_t)s);
}

int launch_patch_128_2_4(const ConvArgs& a, const PatchPlan& p, void* s) {
  return patch::launch_cfg<128, 2, 4>(a, p, (hipStream_t)s);
}

}  // namespace ox
