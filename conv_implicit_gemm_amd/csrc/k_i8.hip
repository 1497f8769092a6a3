// k_i8.hip -- tile-engine instantiations for i8 inputs (Gemm / MatMul
// and convolution); see gemm_conv.hpp.
#include "gemm_conv.hpp"

namespace ox {

int launch_gemm_i8(const GemmArgs& a, int tile, void* stream) {
  return launch_gemm_dt<DT_I8>(a, tile, stream);
}

int launch_conv_i8(const ConvArgs& a, int kind, int tile, void* stream) {
  return launch_conv_dt<DT_I8>(a, kind, tile, stream);
}

}  // namespace ox
