// launch_bf16_d128_trace.hip -- the phase-stamped instances of the 16-bit forward
// kernel for bfloat16 inputs, head dim 128 (the vector-interval accounting).
#define TOS_H16_DEFINE
#include "launch_h16.hpp"

namespace tos {
template hipError_t H16<__bf16, 128>::traced(const FwdArgs&, const KernelChoice&, hipStream_t);
}  // namespace tos
