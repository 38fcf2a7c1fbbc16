// tos_api.hip -- the C ABI of libtos.so (declared in include/tos.h): argument
// validation, kernel selection and launch on the caller's stream.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.hpp"
#include "tos.h"

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810018921;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// TOS_LOG=1 in the environment prints the chosen kernel and HIP errors to stderr
bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("TOS_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

size_t in_elem_bytes(tos_dtype dt) { return dt == TOS_F32 ? 4 : (dt == TOS_FP8_E4M3 ? 1 : 2); }
size_t out_elem_bytes(tos_dtype dt) { return dt == TOS_F32 ? 4 : 2; }

}  // namespace

extern "C" {

int tos_version(void) { return TOS_VERSION; }

const char* tos_status_string(tos_status s) {
  switch (s) {
    case TOS_OK: return "TOS_OK";
    case TOS_ERR_INVALID_ARG: return "TOS_ERR_INVALID_ARG";
    case TOS_ERR_UNSUPPORTED: return "TOS_ERR_UNSUPPORTED";
    case TOS_ERR_HIP: return "TOS_ERR_HIP";
    case TOS_ERR_SCRATCH: return "TOS_ERR_SCRATCH";
  }
  return "TOS_UNKNOWN_STATUS";
}

double tos_attn_fwd_flops(int64_t B, int64_t H, int64_t N, int64_t d, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0.0;
  const double f = 4.0 * (double)B * (double)H * (double)N * (double)N * (double)d;
  return causal ? 0.5 * f : f;
}

tos_status tos_fwd_opts_default(tos_fwd_opts* opts) {
  if (opts == nullptr) return TOS_ERR_INVALID_ARG;
  std::memset(opts, 0, sizeof(*opts));
  opts->size = (int)sizeof(tos_fwd_opts);
  opts->x_tile = 32;
  opts->softmax_split = TOS_SPLIT_VALU;
  opts->fallback = TOS_FALLBACK_OFF;
  opts->fallback_tau = 0.0f;
  opts->q_descale = opts->k_descale = opts->v_descale = 1.0f;
  opts->fallback_tiles = nullptr;
  return TOS_OK;
}

}  // extern "C"

namespace {

// Everything about a call but its pointers: options, sizes and the kernel
// choice.  Returns TOS_OK with *empty set when there is nothing to compute.
tos_status prepare(const tos_fwd_opts* opts, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                   tos_dtype dtype, tos_fwd_opts& op, tos::KernelChoice& kc, bool* empty) {
  *empty = false;
  // ---- options
  tos_fwd_opts_default(&op);
  if (opts != nullptr) {
    if (opts->size != (int)sizeof(tos_fwd_opts)) return TOS_ERR_INVALID_ARG;
    op = *opts;
    if (op.x_tile == 0) op.x_tile = 32;
  }
  if (op.x_tile != 1 && op.x_tile != 16 && op.x_tile != 32 && op.x_tile != 64)
    return TOS_ERR_INVALID_ARG;
  if (op.softmax_split < TOS_SPLIT_VALU || op.softmax_split > TOS_SPLIT_ALL_MFMA)
    return TOS_ERR_INVALID_ARG;
  if (op.split_den < 0 || op.split_num < 0 || op.split_num > op.split_den ||
      (op.split_den == 0 && op.split_num != 0))
    return TOS_ERR_INVALID_ARG;
  if (op.fallback != TOS_FALLBACK_OFF && op.fallback != TOS_FALLBACK_AUTO &&
      op.fallback != TOS_FALLBACK_FORCE)
    return TOS_ERR_INVALID_ARG;
  // tau > 126 would let the switch's rescale exp2(c*(ref - m_i)) overflow fp32
  if (!std::isfinite(op.fallback_tau) || op.fallback_tau < 0.0f || op.fallback_tau > 126.0f)
    return TOS_ERR_INVALID_ARG;
  if (op.schedule != TOS_SCHEDULE_COSCHED && op.schedule != TOS_SCHEDULE_SEQUENTIAL)
    return TOS_ERR_INVALID_ARG;
  if (op.workspace == nullptr && op.workspace_bytes != 0) return TOS_ERR_INVALID_ARG;

  // ---- sizes
  if (dtype != TOS_F32 && dtype != TOS_BF16 && dtype != TOS_FP8_E4M3 && dtype != TOS_F16)
    return TOS_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || N < 0 || d < 0) return TOS_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TOS_ERR_INVALID_ARG;
  if (dtype == TOS_FP8_E4M3) {
    for (float s : {op.q_descale, op.k_descale, op.v_descale})
      if (!std::isfinite(s) || !(s > 0.0f)) return TOS_ERR_INVALID_ARG;
  }
  if (B == 0 || H == 0 || N == 0) {   // nothing to compute
    *empty = true;
    return TOS_OK;
  }
  if (d != 64 && d != 128) return TOS_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  const int64_t nqb = (N + tos::kBr - 1) / tos::kBr;
  // grid size in 32 bits; one head of K or V addressable by a 32-bit buffer offset
  if (B > INT32_MAX || H > INT32_MAX || BH > INT32_MAX || N > INT32_MAX ||
      BH * nqb > INT32_MAX || N * d * (int64_t)in_elem_bytes(dtype) > INT32_MAX)
    return TOS_ERR_UNSUPPORTED;

  // ---- kernel choice
  kc.d = (int)d;
  kc.causal = causal != 0;
  kc.x = op.fallback == TOS_FALLBACK_FORCE ? 1 : op.x_tile;
  kc.fb_auto = op.fallback == TOS_FALLBACK_AUTO && op.x_tile > 1;
  kc.seq = op.schedule == TOS_SCHEDULE_SEQUENTIAL;
  const bool h16 = dtype == TOS_BF16 || dtype == TOS_F16;
  // the matrix unit's share in quarters (the row-sum steps of a key block)
  const bool has_share = op.split_den > 0;
  if (has_share && (4 * op.split_num) % op.split_den != 0) return TOS_ERR_UNSUPPORTED;
  const int quarters = has_share ? 4 * op.split_num / op.split_den : -1;
  // every plan but the vector row sum and the full matrix-unit row sum runs at
  // X = 32 without fallback, co-scheduled, in the 16-bit kernels: the O rescale
  // on the matrix unit needs one alpha per wave
  const bool x32_plain = h16 && op.x_tile == 32 && op.fallback == TOS_FALLBACK_OFF && !kc.seq;
  switch (op.softmax_split) {
    case TOS_SPLIT_VALU:
      if (has_share && quarters != 0) return TOS_ERR_INVALID_ARG;
      kc.plan = tos::kPlanValu;
      break;
    case TOS_SPLIT_ROWSUM_MFMA: {
      const int rs = has_share ? quarters : 4;
      if (dtype == TOS_F32) return TOS_ERR_UNSUPPORTED;
      if (dtype == TOS_FP8_E4M3 && rs != 4) return TOS_ERR_UNSUPPORTED;
      if (rs > 0 && rs < 4 && !x32_plain) return TOS_ERR_UNSUPPORTED;
      kc.plan = tos::split_plan(rs, 0, 0, false);
      break;
    }
    case TOS_SPLIT_SCALE_MFMA:
      if (!x32_plain || (has_share && quarters != 4)) return TOS_ERR_UNSUPPORTED;
      kc.plan = tos::kPlanScaleMfma;
      break;
    case TOS_SPLIT_HSPLIT:
      if (!x32_plain || !has_share || quarters < 1 || quarters > 3) return TOS_ERR_UNSUPPORTED;
      kc.plan = tos::split_plan(quarters, 4 * quarters, 4 * quarters, false);
      break;
    case TOS_SPLIT_VSPLIT:
      if (!x32_plain || !has_share || quarters != 2) return TOS_ERR_UNSUPPORTED;
      kc.plan = tos::split_plan(2, 1, (int)d / 64, true);
      break;
    case TOS_SPLIT_ALL_MFMA:
      if (!x32_plain || (has_share && quarters != 4)) return TOS_ERR_UNSUPPORTED;
      kc.plan = tos::split_plan(4, 16, 16, false);
      break;
  }
  // fp8 sums on the matrix unit whatever the option
  if (dtype == TOS_FP8_E4M3) kc.plan = tos::kPlanValu;
  // the phase-stamped instances
  if (op.trace != nullptr) {
    if (dtype != TOS_BF16 || d != 128 || op.fallback != TOS_FALLBACK_OFF) return TOS_ERR_UNSUPPORTED;
    if (op.trace_bytes < (size_t)tos::device_cus() * tos::kPWaves * tos::kTraceSlots * sizeof(uint64_t))
      return TOS_ERR_INVALID_ARG;
    kc.trace = true;
  } else if (op.trace_bytes != 0) {
    return TOS_ERR_INVALID_ARG;
  }
  if (kc.seq && (!h16 || kc.plan != tos::kPlanValu || kc.fb_auto || kc.x == 16 || kc.x == 64))
    return TOS_ERR_UNSUPPORTED;
  // X = 64 (tiles of two waves): the 16-bit kernels with the vector row sum
  if (kc.x == 64 && (!h16 || kc.plan != tos::kPlanValu)) return TOS_ERR_UNSUPPORTED;

  return TOS_OK;
}

// Pieces for a 16-bit call (pieces.hpp): the piece length in key blocks (0:
// whole query blocks) and the workspace bytes they need.  Only with the
// fallback off: a piece's switch to per-row maxima would be its own.
int split_for(const tos_fwd_opts& op, const tos::KernelChoice& kc, tos_dtype dtype, int64_t BH, int64_t N,
              int64_t d, size_t* bytes) {
  *bytes = 0;
  if ((dtype != TOS_BF16 && dtype != TOS_F16) || op.fallback != TOS_FALLBACK_OFF) return 0;
  const int C = tos::split_blocks((int)BH, (int)N, kc.causal, tos::device_cus());
  if (C <= 0) return 0;
  const int nqb = (int)((N + tos::kPieceRows - 1) / tos::kPieceRows);
  const long long units = tos::units_of((int)BH, nqb, (int)N, kc.causal, C);
  *bytes = (size_t)units * (size_t)tos::piece_bytes((int)d);
  return C;
}

}  // namespace

extern "C" {

tos_status tos_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                       tos_dtype dtype, const tos_fwd_opts* opts, size_t* bytes) {
  if (bytes == nullptr) return TOS_ERR_INVALID_ARG;
  *bytes = 0;
  tos_fwd_opts op;
  tos::KernelChoice kc;
  bool empty = false;
  const tos_status st = prepare(opts, B, H, N, d, causal, dtype, op, kc, &empty);
  if (st != TOS_OK || empty) return st;
  split_for(op, kc, dtype, B * H, N, d, bytes);
  return TOS_OK;
}

tos_status tos_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        tos_dtype dtype, const tos_fwd_opts* opts, void* stream) {
  tos_fwd_opts op;
  tos::KernelChoice kc;
  bool empty = false;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return TOS_ERR_INVALID_ARG;
  const tos_status st = prepare(opts, B, H, N, d, causal, dtype, op, kc, &empty);
  if (st != TOS_OK || empty) return st;
  const int64_t BH = B * H;
  const int64_t nqb = (N + tos::kBr - 1) / tos::kBr;

  // ---- pointers: required, aligned, outputs and workspace overlapping nothing
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return TOS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(op.workspace, 16))
    return TOS_ERR_INVALID_ARG;
  const size_t n_elem = (size_t)BH * (size_t)N * (size_t)d;
  const size_t in_b = n_elem * in_elem_bytes(dtype), out_b = n_elem * out_elem_bytes(dtype);
  const size_t lse_b = lse ? (size_t)BH * (size_t)N * sizeof(float) : 0;
  const size_t ws_b = op.workspace_bytes;
  for (const void* in : {q, k, v}) {
    if (overlaps(o, out_b, in, in_b)) return TOS_ERR_INVALID_ARG;
    if (overlaps(lse, lse_b, in, in_b)) return TOS_ERR_INVALID_ARG;
    if (overlaps(op.workspace, ws_b, in, in_b)) return TOS_ERR_INVALID_ARG;
  }
  if (overlaps(o, out_b, lse, lse_b)) return TOS_ERR_INVALID_ARG;
  if (overlaps(op.workspace, ws_b, o, out_b) || overlaps(op.workspace, ws_b, lse, lse_b))
    return TOS_ERR_INVALID_ARG;
  for (const void* t : {q, k, v, (const void*)o, (const void*)lse, (const void*)op.workspace}) {
    const size_t tb = t == o ? out_b : t == lse ? lse_b : t == op.workspace ? ws_b : in_b;
    if (overlaps(op.trace, op.trace_bytes, t, tb)) return TOS_ERR_INVALID_ARG;
  }

  tos::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)BH;
  a.N = (int)N;
  a.nqb = (int)nqb;
  // fp8: the stored codes times their descales are the real values, so the
  // logit scale takes q_descale * k_descale and O takes v_descale
  const double qk_descale = dtype == TOS_FP8_E4M3 ? (double)op.q_descale * (double)op.k_descale : 1.0;
  a.lse_scale = (float)((double)scale * qk_descale);
  a.c = (float)((double)scale * qk_descale * kLog2e);
  a.o_scale = dtype == TOS_FP8_E4M3 ? op.v_descale : 1.0f;
  // default thresholds: bf16/fp32 P~ keep 2^-100 far above their underflow;
  // e4m3 P~ (pre-scaled by 2^8) keeps every row's largest term >= 2^-4; fp16
  // P~ (pre-scaled by 2^15) keeps it >= 2^-9, a normal number
  a.tau = op.fallback_tau > 0.0f ? op.fallback_tau
                                 : (dtype == TOS_FP8_E4M3 ? 12.0f : (dtype == TOS_F16 ? 24.0f : 100.0f));
  a.fallback_tiles = op.fallback_tiles;
  // FORCE runs the per-row kernel and counts every X-row tile of the request
  a.count_x = op.fallback == TOS_FALLBACK_FORCE ? op.x_tile : 0;
  if (op.fallback == TOS_FALLBACK_AUTO && op.x_tile == 1) a.count_x = 0;

  // pieces of query blocks, when the workspace holds them
  a.split_c = 0;
  a.ws = nullptr;
  size_t need = 0;
  const int C = split_for(op, kc, dtype, BH, N, d, &need);
  if (C > 0 && op.workspace != nullptr && op.workspace_bytes >= need) {
    a.split_c = C;
    a.ws = (float*)op.workspace;
  }
  a.nunits = (int)(BH * nqb);
  a.trace = (unsigned long long*)op.trace;

  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipErrorNotSupported;
  if (dtype == TOS_BF16)
    e = tos::launch_bf16(a, kc, s);
  else if (dtype == TOS_F16)
    e = tos::launch_f16(a, kc, s);
  else if (dtype == TOS_F32)
    e = tos::launch_f32(a, kc, s);
  else
    e = tos::launch_fp8(a, kc, s);
  if (log_enabled())
    std::fprintf(stderr, "[tos] dtype=%d B=%lld H=%lld N=%lld d=%d causal=%d X=%d plan=0x%x "
                 "fallback=%d sequential=%d items=%lld pieces=%d: %s\n", (int)dtype, (long long)B, (long long)H,
                 (long long)N, kc.d, (int)kc.causal, kc.x, kc.plan, op.fallback,
                 (int)kc.seq, (long long)(BH * nqb), a.split_c, hipGetErrorString(e));
  if (e == hipErrorNotSupported) return TOS_ERR_UNSUPPORTED;
  return e == hipSuccess ? TOS_OK : TOS_ERR_HIP;
}

}  // extern "C"
