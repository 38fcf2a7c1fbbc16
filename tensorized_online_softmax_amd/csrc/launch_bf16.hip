// launch_bf16.hip -- the 16-bit forward kernel for bfloat16 inputs.
#include "launch_h16.hpp"

namespace tos {

hipError_t launch_bf16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return launch_h16<__bf16>(a, k, s);
}

}  // namespace tos
