// launch.hpp -- internal: per-dtype launchers behind the C ABI (tos_api.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>

#include "attn_fwd_kernels.hpp"

namespace tos {

struct KernelChoice {
  int d;             // 64 or 128
  bool causal;
  int x;             // 1, 16, 32 or 64
  int plan = 0;      // split plan (split_plan in attn_fwd_kernels.hpp): 16-bit
                     // kernels; fp8 always sums on the matrix unit, fp32 never
  bool fb_auto;      // fallback AUTO (x > 1 only)
  bool seq = false;  // sequential schedule (16-bit kernels, x = 1 or 32, vector row sum, no AUTO)
  bool trace = false;   // the phase-stamped instances (bf16, d = 128, the ablation's settings)
};

// Workgroups of a persistent launch over `nitems` items: one per compute unit
// of the current device (the kernels fill a compute unit with one workgroup),
// rounded down to a multiple of 8 (the XCD count) when there are more items
// than compute units.  The count is read once per device.
// Compute units of the current device, read once per device (256 when the
// runtime cannot say).
inline int device_cus() {
  static std::atomic<int> cus[64];   // 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  int n = dev >= 0 ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    if (dev >= 0) cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

inline int persistent_grid(int nitems) {
  const int n = device_cus();
  if (nitems <= n) return nitems;
  return n >= 8 ? n & ~7 : n;
}

// Pieces per item for a 16-bit launch of BH heads (pieces.hpp): 0 (whole
// items) when there are at least as many items as compute units; else the
// shortest piece length C >= kMinPieceBlocks whose units number at most
// min(compute units, kMaxPieces), or 0 when no item would be cut.
inline int split_blocks(int BH, int N, bool causal, int cus) {
  const int nqb = (N + kPieceRows - 1) / kPieceRows;
  const long long items = (long long)BH * nqb;
  const int cap = cus < kMaxPieces ? cus : kMaxPieces;
  if (items >= cap) return 0;
  long long total = 0;
  int longest = 0;
  for (int qb = 0; qb < nqb; ++qb) {
    const int n = qblock_blocks(qb, N, causal);
    total += (long long)BH * n;
    longest = n > longest ? n : longest;
  }
  long long c = (total + cap - 1) / cap;
  if (c < kMinPieceBlocks) c = kMinPieceBlocks;
  for (; c < longest; ++c)
    if (units_of(BH, nqb, N, causal, (int)c) <= cap) return (int)c;
  return 0;
}

// Each returns hipSuccess, hipErrorNotSupported for a combination that has no
// instance, or the launch error.
hipError_t launch_bf16(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_f16(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_f32(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);
hipError_t launch_fp8(const FwdArgs& a, const KernelChoice& k, hipStream_t stream);

}  // namespace tos
