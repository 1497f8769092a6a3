// k_conv_pw_b.hip -- 128-channel configurations of the pointwise kernel
// (2 x 2 waves: 128 channels x 128 pixels per block).
#include "conv_pw.hpp"

namespace ox {

int launch_pw_2_32(const ConvArgs& a, const PwPlan& p, void* s) {
  return pw::launch_cfg<2, 2, 32>(a, p, (hipStream_t)s);
}

int launch_pw_2_64(const ConvArgs& a, const PwPlan& p, void* s) {
  return pw::launch_cfg<2, 2, 64>(a, p, (hipStream_t)s);
}

}  // namespace ox
