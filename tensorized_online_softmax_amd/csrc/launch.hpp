// launch.hpp -- internal: per-dtype launchers behind the C ABI (tos_api.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "attn_fwd_kernels.hpp"

namespace tos {

struct KernelChoice {
  int d;             // 64 or 128
  bool causal;
  int x;             // 1, 16 or 32
  bool rowsum_mfma;  // row sum on the matrix unit (fp8: always)
  bool fb_auto;      // fallback AUTO (x > 1 only)
};

// Each returns hipSuccess, hipErrorNotSupported for a combination that has no
// instance, or the launch error.
hipError_t launch_bf16(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_f16(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_f32(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_fp8(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);

}  // namespace tos
