// launch_f16_d64_main.hip -- the 16-bit forward kernel's main instances for float16 inputs, head dim 64.
#define TOS_H16_DEFINE
#include "launch_h16.hpp"

namespace tos {
template hipError_t H16<_Float16, 64>::main(const FwdArgs&, const KernelChoice&, hipStream_t);
}  // namespace tos
