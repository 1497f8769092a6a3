// k_conv_pw_a.hip -- 64-channel configurations of the pointwise kernel
// (1 x 4 waves: 64 channels x 256 pixels per block).
#include "conv_pw.hpp"

namespace ox {

int launch_pw_1_32(const ConvArgs& a, const PwPlan& p, void* s) {
  return pw::launch_cfg<1, 4, 32>(a, p, (hipStream_t)s);
}

int launch_pw_1_64(const ConvArgs& a, const PwPlan& p, void* s) {
  return pw::launch_cfg<1, 4, 64>(a, p, (hipStream_t)s);
}

}  // namespace ox
