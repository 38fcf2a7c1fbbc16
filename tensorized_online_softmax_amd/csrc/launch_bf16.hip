// launch_bf16.hip -- instances and launcher of the bf16 forward kernel.
#include "launch.hpp"

namespace tos {

template <int D, bool CAUSAL, int X, bool RS, bool FB>
static hipError_t go(const FwdArgs& a, hipStream_t s) {
  FwdArgs arg = a;
  arg.nqb = (a.N + kPBr - 1) / kPBr;
  const dim3 grid((unsigned)arg.BH * (unsigned)arg.nqb), block(kPThreads);
  // hipLaunchKernel reports this launch's own status (hipGetLastError could
  // return an error left behind by an earlier, unrelated call)
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_bf16<D, CAUSAL, X, RS, FB>), grid, block, params, 0, s);
}

template <int D, bool CAUSAL>
static hipError_t by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.x == 1) {
    if (k.fb_auto) return hipErrorNotSupported;
    return k.rowsum_mfma ? go<D, CAUSAL, 1, true, false>(a, s) : go<D, CAUSAL, 1, false, false>(a, s);
  }
  if (k.x == 16) {
    if (k.rowsum_mfma)
      return k.fb_auto ? go<D, CAUSAL, 16, true, true>(a, s) : go<D, CAUSAL, 16, true, false>(a, s);
    return k.fb_auto ? go<D, CAUSAL, 16, false, true>(a, s) : go<D, CAUSAL, 16, false, false>(a, s);
  }
  if (k.x == 32) {
    if (k.rowsum_mfma)
      return k.fb_auto ? go<D, CAUSAL, 32, true, true>(a, s) : go<D, CAUSAL, 32, true, false>(a, s);
    return k.fb_auto ? go<D, CAUSAL, 32, false, true>(a, s) : go<D, CAUSAL, 32, false, false>(a, s);
  }
  return hipErrorNotSupported;
}

hipError_t launch_bf16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.d == 64) return k.causal ? by_x<64, true>(a, k, s) : by_x<64, false>(a, k, s);
  if (k.d == 128) return k.causal ? by_x<128, true>(a, k, s) : by_x<128, false>(a, k, s);
  return hipErrorNotSupported;
}

}  // namespace tos
