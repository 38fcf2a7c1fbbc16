// launch_f32.hip -- instances and launcher of the fp32 forward kernels: 128-row
// workgroups, or 16-row slabs whose keys are split across the workgroup's waves
// (and whose head dim is shared among up to 4 workgroups) when the 128-row grid
// would leave compute units idle.
#include "attn_fwd_f32_slab.hpp"
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

template <int D, bool CAUSAL, int X, int DS>
static hipError_t go_slab(const FwdArgs& a, long long slabs, hipStream_t s) {
  const dim3 grid((unsigned)(slabs * DS)), block(kSlabThreads);
  FwdArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_f32_slab<D, CAUSAL, X, DS>), grid, block, params, 0,
                         s);
}

// slabs over DS shares of the head dim: the most shares whose grid still fits
// the compute units (each share repeats the slab's S work on an idle unit)
template <int D, bool CAUSAL, int X>
static hipError_t by_share(const FwdArgs& a, hipStream_t s) {
  const long long slabs = (long long)a.BH * ((a.N + kSlabRows - 1) / kSlabRows);
  const int cus = device_cus();
  if (4 * slabs <= cus) return go_slab<D, CAUSAL, X, 4>(a, slabs, s);
  if (2 * slabs <= cus) return go_slab<D, CAUSAL, X, 2>(a, slabs, s);
  return go_slab<D, CAUSAL, X, 1>(a, slabs, s);
}

template <int D, bool CAUSAL>
static hipError_t by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.plan != kPlanValu) return hipErrorNotSupported;
  // slabs: X = 1 or 16 without the fallback switch or the tile count, when the
  // 128-row workgroups number fewer than the compute units
  const long long nqb = (a.N + kBr - 1) / kBr;
  if ((k.x == 1 || k.x == 16) && !k.fb_auto && a.count_x == 0 && (long long)a.BH * nqb < device_cus())
    return k.x == 1 ? by_share<D, CAUSAL, 1>(a, s) : by_share<D, CAUSAL, 16>(a, s);
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
