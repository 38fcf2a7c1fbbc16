// launch_f16.hip -- the 16-bit forward kernel for float16 inputs.
#include "launch_h16.hpp"

namespace tos {

hipError_t launch_f16(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return launch_h16<_Float16>(a, k, s);
}

}  // namespace tos
