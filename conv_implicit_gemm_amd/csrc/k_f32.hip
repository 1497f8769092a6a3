// k_f32.hip -- tile-engine instantiations for f32 inputs (Gemm / MatMul
// and convolution); see gemm_conv.hpp.
#include "gemm_conv.hpp"

namespace ox {

int launch_gemm_f32(const GemmArgs& a, int tile, void* stream) {
  return launch_gemm_dt<DT_F32>(a, tile, stream);
}

int launch_conv_f32(const ConvArgs& a, int kind, int tile, void* stream) {
  return launch_conv_dt<DT_F32>(a, kind, tile, stream);
}

int launch_gemm_splitk_f32(const GemmArgs& a, int S, int kslice, float* ws, void* stream) {
  return launch_gemm_splitk_dt<DT_F32>(a, S, kslice, ws, stream);
}

}  // namespace ox
