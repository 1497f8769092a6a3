// k_conv_pwd.hip -- configurations of the DMA-staged pointwise kernel.
// launch_pwd_<BP>_<BC>_<KC>: BP pixels x BC output channels per block, KC
// input channels per ring stage (the ring depth and wave layout follow).
#include "conv_pwd.hpp"

namespace ox {

int launch_pwd_128_64_64(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<128, 64, 64, 3, 4>(a, p, (hipStream_t)s);
}
int launch_pwd_128_64_32(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<128, 64, 32, 4, 4>(a, p, (hipStream_t)s);
}
int launch_pwd_64_64_64(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<64, 64, 64, 4, 2>(a, p, (hipStream_t)s);
}
int launch_pwd_64_128_64(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<64, 128, 64, 3, 2>(a, p, (hipStream_t)s);
}
int launch_pwd_64_128_32(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<64, 128, 32, 4, 2>(a, p, (hipStream_t)s);
}
int launch_pwd_64_256_64(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<64, 256, 64, 2, 1>(a, p, (hipStream_t)s);
}
int launch_pwd_64_256_32(const ConvArgs& a, const PwdPlan& p, void* s) {
  return pwd::launch<64, 256, 32, 3, 1>(a, p, (hipStream_t)s);
}

}  // namespace ox
