// launch_h16.hpp -- instances and launcher of the 16-bit (bf16 / fp16) forward
// kernel, for one element type per translation unit.
#pragma once
#include "launch.hpp"

namespace tos {

template <typename E, int D, bool CAUSAL, int X, bool RS, bool FB, bool SEQ = false, bool SCALE = false>
static hipError_t go_h16(const FwdArgs& a, hipStream_t s) {
  FwdArgs arg = a;
  arg.nqb = (a.N + kPBr - 1) / kPBr;
  const dim3 grid((unsigned)persistent_grid(arg.BH * arg.nqb)), block(kPThreads);
  // hipLaunchKernel reports this launch's own status (hipGetLastError could
  // return an error left behind by an earlier, unrelated call)
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_h16<E, D, CAUSAL, X, RS, FB, SEQ, SCALE>), grid,
                         block, params, 0, s);
}

template <typename E, int D, bool CAUSAL>
static hipError_t by_x_h16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.scale_mfma) {   // the O rescale on the matrix unit: X = 32, VALU row sum, no AUTO
    if (k.x != 32 || k.rowsum_mfma || k.fb_auto || k.seq) return hipErrorNotSupported;
    return go_h16<E, D, CAUSAL, 32, false, false, false, true>(a, s);
  }
  if (k.seq) {   // the sequential-schedule ablation: VALU row sum, no AUTO
    if (k.rowsum_mfma || k.fb_auto) return hipErrorNotSupported;
    if (k.x == 1) return go_h16<E, D, CAUSAL, 1, false, false, true>(a, s);
    if (k.x == 32) return go_h16<E, D, CAUSAL, 32, false, false, true>(a, s);
    return hipErrorNotSupported;
  }
  if (k.x == 1) {
    if (k.fb_auto) return hipErrorNotSupported;
    return k.rowsum_mfma ? go_h16<E, D, CAUSAL, 1, true, false>(a, s) : go_h16<E, D, CAUSAL, 1, false, false>(a, s);
  }
  if (k.x == 16) {
    if (k.rowsum_mfma)
      return k.fb_auto ? go_h16<E, D, CAUSAL, 16, true, true>(a, s) : go_h16<E, D, CAUSAL, 16, true, false>(a, s);
    return k.fb_auto ? go_h16<E, D, CAUSAL, 16, false, true>(a, s) : go_h16<E, D, CAUSAL, 16, false, false>(a, s);
  }
  if (k.x == 64) {   // tiles of two waves: VALU row sum only
    if (k.rowsum_mfma) return hipErrorNotSupported;
    return k.fb_auto ? go_h16<E, D, CAUSAL, 64, false, true>(a, s) : go_h16<E, D, CAUSAL, 64, false, false>(a, s);
  }
  if (k.x == 32) {
    if (k.rowsum_mfma)
      return k.fb_auto ? go_h16<E, D, CAUSAL, 32, true, true>(a, s) : go_h16<E, D, CAUSAL, 32, true, false>(a, s);
    return k.fb_auto ? go_h16<E, D, CAUSAL, 32, false, true>(a, s) : go_h16<E, D, CAUSAL, 32, false, false>(a, s);
  }
  return hipErrorNotSupported;
}

template <typename E>
static hipError_t launch_h16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.d == 64) return k.causal ? by_x_h16<E, 64, true>(a, k, s) : by_x_h16<E, 64, false>(a, k, s);
  if (k.d == 128) return k.causal ? by_x_h16<E, 128, true>(a, k, s) : by_x_h16<E, 128, false>(a, k, s);
  return hipErrorNotSupported;
}

}  // namespace tos
