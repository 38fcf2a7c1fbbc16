// launch_h16.hpp -- instances and launchers of the 16-bit (bf16 / fp16)
// forward kernel.  H16<E, D>::main holds the instances every caller may pick
// (X = 1 / 16 / 32 / 64, vector or matrix-unit row sum, fallback off / auto);
// H16<E, D>::ablation the ablation settings (sequential schedule, partial row
// sums and the other split plans at X = 32).  Each (element type, head dim,
// group) is instantiated in its own translation unit, so that they compile in
// parallel; launch_h16.hip dispatches.
#pragma once
#include "launch.hpp"

namespace tos {

template <typename E, int D>
struct H16 {
  static hipError_t main(const FwdArgs& a, const KernelChoice& k, hipStream_t s);
  static hipError_t ablation(const FwdArgs& a, const KernelChoice& k, hipStream_t s);
  static hipError_t traced(const FwdArgs& a, const KernelChoice& k, hipStream_t s);
};

// Is this choice one of the ablation instances?
inline bool h16_is_ablation(const KernelChoice& k) {
  return k.seq || (k.plan != kPlanValu && k.plan != kPlanRowsumMfma);
}

#ifdef TOS_H16_DEFINE
template <typename E, int D, bool CAUSAL, int X, int PLAN, bool FB, bool SEQ = false, bool TRACE = false>
static hipError_t go_h16(const FwdArgs& a, hipStream_t s) {
  FwdArgs arg = a;
  arg.nqb = (a.N + kPBr - 1) / kPBr;
  arg.nunits = (int)units_of(arg.BH, arg.nqb, arg.N, CAUSAL, arg.split_c);
  const dim3 grid((unsigned)persistent_grid(arg.nunits)), block(kPThreads);
  // hipLaunchKernel reports this launch's own status (hipGetLastError could
  // return an error left behind by an earlier, unrelated call)
  void* params[] = {&arg};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_h16<E, D, CAUSAL, X, PLAN, FB, SEQ, TRACE>),
                                 grid, block, params, 0, s);
  if (e != hipSuccess || arg.split_c <= 0) return e;
  // the pieces' partial results, merged per item on the same stream
  const unsigned wgs = (unsigned)(arg.BH * arg.nqb) * (unsigned)(kPieceRows / kMergeRowsPerWg<D>);
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_merge_h16<E, D, CAUSAL>), dim3(wgs), dim3(256),
                         params, 0, s);
}

template <typename E, int D, bool CAUSAL>
static hipError_t main_by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  constexpr int V = kPlanValu, R = kPlanRowsumMfma;
  const bool rs = k.plan == R;
  if (k.plan != V && k.plan != R) return hipErrorNotSupported;
  if (k.x == 1) {
    if (k.fb_auto) return hipErrorNotSupported;
    return rs ? go_h16<E, D, CAUSAL, 1, R, false>(a, s) : go_h16<E, D, CAUSAL, 1, V, false>(a, s);
  }
  if (k.x == 16) {
    if (rs) return k.fb_auto ? go_h16<E, D, CAUSAL, 16, R, true>(a, s) : go_h16<E, D, CAUSAL, 16, R, false>(a, s);
    return k.fb_auto ? go_h16<E, D, CAUSAL, 16, V, true>(a, s) : go_h16<E, D, CAUSAL, 16, V, false>(a, s);
  }
  if (k.x == 32) {
    if (rs) return k.fb_auto ? go_h16<E, D, CAUSAL, 32, R, true>(a, s) : go_h16<E, D, CAUSAL, 32, R, false>(a, s);
    return k.fb_auto ? go_h16<E, D, CAUSAL, 32, V, true>(a, s) : go_h16<E, D, CAUSAL, 32, V, false>(a, s);
  }
  if (k.x == 64) {   // tiles of two waves: vector row sum only
    if (rs) return hipErrorNotSupported;
    return k.fb_auto ? go_h16<E, D, CAUSAL, 64, V, true>(a, s) : go_h16<E, D, CAUSAL, 64, V, false>(a, s);
  }
  return hipErrorNotSupported;
}

// the split plans of the ablation, all at X = 32 without fallback (the O
// rescale on the matrix unit needs one alpha per wave)
template <int D> constexpr int kAblationPlans[] = {
    split_plan(1, 0, 0, false),   // row sum: 1 of 4 steps on the matrix unit
    split_plan(2, 0, 0, false),   //          2 of 4
    split_plan(3, 0, 0, false),   //          3 of 4
    kPlanScaleMfma,               // O rescale only
    split_plan(1, 4, 4, false),   // horizontal split 1/4
    split_plan(2, 8, 8, false),   //                  1/2
    split_plan(3, 12, 12, false), //                  3/4
    split_plan(2, 1, D / 64, true),   // vertical split 1/2: S tile 0, half the O tiles
    split_plan(4, 16, 16, false), // everything on the matrix unit
};

template <typename E, int D, bool CAUSAL, int I = 0>
static hipError_t abl_plan(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  constexpr int n = sizeof(kAblationPlans<D>) / sizeof(int);
  if constexpr (I == n) {
    return hipErrorNotSupported;
  } else {
    if (k.plan == kAblationPlans<D>[I]) return go_h16<E, D, CAUSAL, 32, kAblationPlans<D>[I], false>(a, s);
    return abl_plan<E, D, CAUSAL, I + 1>(a, k, s);
  }
}

template <typename E, int D, bool CAUSAL>
static hipError_t abl_by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  if (k.seq) {   // the sequential-schedule ablation: vector row sum, no AUTO
    if (k.plan != kPlanValu || k.fb_auto) return hipErrorNotSupported;
    if (k.x == 1) return go_h16<E, D, CAUSAL, 1, kPlanValu, false, true>(a, s);
    if (k.x == 32) return go_h16<E, D, CAUSAL, 32, kPlanValu, false, true>(a, s);
    return hipErrorNotSupported;
  }
  if (k.x != 32 || k.fb_auto) return hipErrorNotSupported;
  return abl_plan<E, D, CAUSAL>(a, k, s);
}

// the phase-stamped instances: the settings of the vector-interval table
// (per-row and tile-32 sequential, per-row, tile-16 and tile-32 co-scheduled,
// matrix-unit row sum, everything on the matrix unit), fallback off
template <typename E, int D, bool CAUSAL>
static hipError_t traced_by_x(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  constexpr int V = kPlanValu, R = kPlanRowsumMfma, A = split_plan(4, 16, 16, false);
  if (k.fb_auto) return hipErrorNotSupported;
  if (k.seq) {
    if (k.plan != V) return hipErrorNotSupported;
    if (k.x == 1) return go_h16<E, D, CAUSAL, 1, V, false, true, true>(a, s);
    if (k.x == 32) return go_h16<E, D, CAUSAL, 32, V, false, true, true>(a, s);
    return hipErrorNotSupported;
  }
  if (k.x == 1 && k.plan == V) return go_h16<E, D, CAUSAL, 1, V, false, false, true>(a, s);
  if (k.x == 16 && k.plan == V) return go_h16<E, D, CAUSAL, 16, V, false, false, true>(a, s);
  if (k.x == 32 && k.plan == V) return go_h16<E, D, CAUSAL, 32, V, false, false, true>(a, s);
  if (k.x == 32 && k.plan == R) return go_h16<E, D, CAUSAL, 32, R, false, false, true>(a, s);
  if (k.x == 32 && k.plan == A) return go_h16<E, D, CAUSAL, 32, A, false, false, true>(a, s);
  return hipErrorNotSupported;
}

template <typename E, int D>
hipError_t H16<E, D>::traced(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return k.causal ? traced_by_x<E, D, true>(a, k, s) : traced_by_x<E, D, false>(a, k, s);
}

template <typename E, int D>
hipError_t H16<E, D>::main(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return k.causal ? main_by_x<E, D, true>(a, k, s) : main_by_x<E, D, false>(a, k, s);
}
template <typename E, int D>
hipError_t H16<E, D>::ablation(const FwdArgs& a, const KernelChoice& k, hipStream_t s) {
  return k.causal ? abl_by_x<E, D, true>(a, k, s) : abl_by_x<E, D, false>(a, k, s);
}
#endif  // TOS_H16_DEFINE

}  // namespace tos
