// launch_f32.hip -- instances and launcher of the fp32 forward kernel.
#include "launch.hpp"

namespace tos {

template <int D, bool CAUSAL, int X, bool FB>
static hipError_t go(const FwdArgs& a, hipStream_t s) {
  FwdArgs arg = a;
  arg.nqb = (a.N + kBr - 1) / kBr;
  const dim3 grid((unsigned)arg.BH * (unsigned)arg.nqb), block(kThreads);
  // hipLaunchKernel reports this launch's own status (hipGetLastError could
  // return an error left behind by an earlier, unrelated call)
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_f32<D, CAUSAL, X, FB>), grid, block, params, 0, s);
}

template <int D, bool CAUSAL>
static hipError_t by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.plan != kPlanValu) return hipErrorNotSupported;
  if (k.x == 1) return k.fb_auto ? hipErrorNotSupported : go<D, CAUSAL, 1, false>(a, s);
  if (k.x == 16) return k.fb_auto ? go<D, CAUSAL, 16, true>(a, s) : go<D, CAUSAL, 16, false>(a, s);
  if (k.x == 32) return k.fb_auto ? go<D, CAUSAL, 32, true>(a, s) : go<D, CAUSAL, 32, false>(a, s);
  return hipErrorNotSupported;
}

hipError_t launch_f32(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.d == 64) return k.causal ? by_x<64, true>(a, k, s) : by_x<64, false>(a, k, s);
  if (k.d == 128) return k.causal ? by_x<128, true>(a, k, s) : by_x<128, false>(a, k, s);
  return hipErrorNotSupported;
}

}  // namespace tos
