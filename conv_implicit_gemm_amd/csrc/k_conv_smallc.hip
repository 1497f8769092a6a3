// k_conv_smallc.hip -- launchers of the few-input-channel kernel.
#include "conv_smallc.hpp"

namespace ox {

namespace {

template <int S, int NH, int FP>
void launch_p(const ConvArgs& a, const SmallcPlan& p, hipStream_t s) {
  dim3 grid(p.nrb * a.N * p.nmb, 1, 1);
  if (p.P == 8)
    hipLaunchKernelGGL((smallc::conv_smallc_bf16<S, NH, FP, 8>), grid, dim3(kThreads), p.lds, s, a, p);
  else
    hipLaunchKernelGGL((smallc::conv_smallc_bf16<S, NH, FP, 1>), grid, dim3(kThreads), p.lds, s, a, p);
}

template <int S, int NH>
void launch_fp(const ConvArgs& a, const SmallcPlan& p, hipStream_t s) {
  if (p.FP == 4) launch_p<S, NH, 4>(a, p, s);
  else launch_p<S, NH, 2>(a, p, s);
}

}  // namespace

int launch_smallc(const ConvArgs& a, const SmallcPlan& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.sh == 2) {
    if (p.NH == 2) launch_fp<2, 2>(a, p, s);
    else launch_fp<2, 1>(a, p, s);
  } else {
    if (p.NH == 2) launch_fp<1, 2>(a, p, s);
    else launch_fp<1, 1>(a, p, s);
  }
  return (int)hipGetLastError();
}

}  // namespace ox
