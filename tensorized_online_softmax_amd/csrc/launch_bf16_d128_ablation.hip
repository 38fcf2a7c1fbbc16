// launch_bf16_d128_ablation.hip -- the 16-bit forward kernel's ablation instances for bfloat16 inputs, head dim 128.
#define TOS_H16_DEFINE
#include "launch_h16.hpp"

namespace tos {
template hipError_t H16<__bf16, 128>::ablation(const FwdArgs&, const KernelChoice&, hipStream_t);
}  // namespace tos
