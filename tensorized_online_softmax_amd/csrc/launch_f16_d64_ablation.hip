// launch_f16_d64_ablation.hip -- the 16-bit forward kernel's ablation instances for float16 inputs, head dim 64.
#define TOS_H16_DEFINE
#include "launch_h16.hpp"

namespace tos {
template hipError_t H16<_Float16, 64>::ablation(const FwdArgs&, const KernelChoice&, hipStream_t);
}  // namespace tos
