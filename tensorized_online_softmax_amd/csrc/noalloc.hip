// noalloc.hip -- tos_attn_fwd_noalloc: tos_attn_fwd for callers that cannot
// allocate device memory.  The workspace of the key pieces (pieces.hpp) is a
// file-scope device array of the largest size any call can need, whose
// address is looked up once per device.
#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "tos.h"

namespace {

// 256 units x 256 rows x (2 x 128 + 8) bytes: the most the pieces of any call
// use (at most kMaxPieces units, d <= 128)
constexpr size_t kScratchBytes = (size_t)tos::kMaxPieces * (size_t)tos::piece_bytes(128);

// Device storage of each GPU the library runs on (held until the process
// ends).  In host code this name is only a stand-in: its device address comes
// from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// The current device's copy of the array, or nullptr if the runtime cannot
// say where it is.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" tos_status tos_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                           int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                           float scale, tos_dtype dtype, const tos_fwd_opts* opts,
                                           void* stream) {
  tos_fwd_opts op;
  if (tos_fwd_opts_default(&op) != TOS_OK) return TOS_ERR_INVALID_ARG;
  if (opts != nullptr) {
    if (opts->size != (int)sizeof(tos_fwd_opts)) return TOS_ERR_INVALID_ARG;
    op = *opts;
  }
  // the workspace is the library's own here
  if (op.workspace != nullptr || op.workspace_bytes != 0) return TOS_ERR_INVALID_ARG;
  size_t need = 0;
  const tos_status st = tos_attn_fwd_workspace_size(B, H, N, d, causal, dtype, &op, &need);
  if (st != TOS_OK) return st;
  if (need > kScratchBytes) return TOS_ERR_SCRATCH;
  if (need > 0) {
    void* ws = device_scratch();
    if (ws == nullptr) return TOS_ERR_HIP;
    op.workspace = ws;
    op.workspace_bytes = kScratchBytes;
  }
  return tos_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, &op, stream);
}
