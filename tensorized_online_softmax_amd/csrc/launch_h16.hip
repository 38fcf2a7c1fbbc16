// launch_h16.hip -- dispatch of the 16-bit forward kernel (bf16, fp16) to the
// translation unit that holds the chosen instance.
#include "launch_h16.hpp"

namespace tos {

template <typename E>
static hipError_t launch_h16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.trace) {   // phase-stamped instances: bf16, d = 128
    if constexpr (__is_same(E, __bf16)) {
      if (k.d == 128) return H16<E, 128>::traced(a, k, s);
    }
    return hipErrorNotSupported;
  }
  const bool abl = h16_is_ablation(k);
  if (k.d == 64) return abl ? H16<E, 64>::ablation(a, k, s) : H16<E, 64>::main(a, k, s);
  if (k.d == 128) return abl ? H16<E, 128>::ablation(a, k, s) : H16<E, 128>::main(a, k, s);
  return hipErrorNotSupported;
}

hipError_t launch_bf16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return launch_h16<__bf16>(a, k, s);
}
hipError_t launch_f16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return launch_h16<_Float16>(a, k, s);
}

}  // namespace tos
