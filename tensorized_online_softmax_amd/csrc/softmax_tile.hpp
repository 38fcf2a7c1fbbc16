// softmax_tile.hpp -- per-lane state of the tensorized online softmax (gfx950).
//
// Layout these helpers assume (the 32x32 MFMA accumulator layout of S^T = K Q^T):
// lane L of a 64-wide wave owns query (L mod 32) of the wave's 32 queries; lanes
// L and L+32 hold different keys of the same query.  So a row's statistics are
// combined across the lane pair (L, L+32), and an X-row tile (X = 16 or 32) is a
// set of X consecutive lanes mod 32.  (X = 64 spans two waves; the kernels
// combine the two 32-row halves.)
//
// The surrogate maximum (FlashAttention-T, section A2, "surrogate maximum"): the
// reference subtracted from a row's logits is the largest running row maximum
// over the row's X-row tile; with X = 1 it is the row's own running maximum.
// Optional fallback (section A2, "numerical stability guarantees"): a tile whose
// gap c*(m^ - min_i m_i) exceeds tau switches to per-row maxima for good.
#pragma once
#include <hip/hip_runtime.h>

namespace tos {

__device__ __forceinline__ float fmax_raw(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ float fmin_raw(float a, float b) { return __builtin_fminf(a, b); }
// max(a, b, c) as one v_max3_f32 (finite inputs)
__device__ __forceinline__ float fmax3_raw(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float m;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(a), "v"(b), "v"(c));
  return m;
#else
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
#endif
}

// value of the other lane of the pair (L, L xor 32), combined with op
template <typename Op>
__device__ __forceinline__ float pair_reduce(float x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// reduce over the 16 lanes of each DPP row: pairs, quads, half-rows, rows
template <typename Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {
  x = op(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp<0x141>(x));   // row_half_mirror
  x = op(x, dpp<0x140>(x));   // row_mirror
  return x;
}

// reduce over the X lanes (mod 32) of a tile; input must already agree across
// the lane pair (L, L+32)
template <int X, typename Op>
__device__ __forceinline__ float tile_reduce(float x, Op op) {
  static_assert(X == 1 || X == 16 || X == 32, "tile rows");
  if constexpr (X == 1) {
    return x;
  } else {
    x = row16_reduce(x, op);
    if constexpr (X == 32) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
  }
}

struct MaxOp { __device__ float operator()(float a, float b) const { return fmax_raw(a, b); } };
struct MinOp { __device__ float operator()(float a, float b) const { return fmin_raw(a, b); } };

// Per-lane softmax state of one query row.
struct RowState {
  float m_run;     // running row maximum of the raw logits (-inf: no key yet)
  float ref;       // reference maximum the exponentials are taken against
  bool per_row;    // this lane's tile uses per-row maxima (fallback)
};

__device__ __forceinline__ void row_state_init(RowState& st, bool per_row) {
  st.m_run = -__builtin_inff();
  st.ref = -__builtin_inff();
  st.per_row = per_row;
}

// Algorithm 1 step 1 (tile max) and the reference update for one key block,
// in three parts so that callers can spread them between matrix instructions.
// `blk_max` is this lane's maximum over its logits of the block (before the
// pair combine).
__device__ __forceinline__ void row_max_update(RowState& st, float blk_max) {
  st.m_run = fmax_raw(st.m_run, pair_reduce(blk_max, MaxOp()));
}

// The block's reference: the tile maximum of the running row maxima (the
// surrogate), or the row's own maximum once its tile went per-row.
// Straight-line code (selects, no branches), so that the caller's matrix
// instructions can be interleaved with it in one basic block.
template <int X, bool FB_AUTO>
__device__ __forceinline__ float block_ref(RowState& st, float c, float tau) {
  if constexpr (X == 1) {
    return st.m_run;
  } else {
    const float tm = tile_reduce<X>(st.m_run, MaxOp());
    if constexpr (FB_AUTO) {
      // rows without a key yet cannot underflow: leave them out of the min
      const float ninf = -__builtin_inff();
      const float mn = tile_reduce<X>(st.m_run == ninf ? __builtin_inff() : st.m_run, MinOp());
      st.per_row = st.per_row || (c * (tm - mn) > tau);
      return st.per_row ? st.m_run : tm;
    } else {
      return tm;
    }
  }
}

// The same reference from a tile's maximum tm and minimum mn of the running row
// maxima (rows without a key left out of mn), for tiles that span two waves.
template <bool FB_AUTO>
__device__ __forceinline__ float ref_from_tile(RowState& st, float tm, float mn, float c, float tau) {
  if constexpr (FB_AUTO) {
    st.per_row = st.per_row || (c * (tm - mn) > tau);
    return st.per_row ? st.m_run : tm;
  } else {
    return tm;
  }
}

// Moves the reference to ref_new.  Returns alpha = exp2(c*(ref_old - ref_new)):
// 0 when nothing was accumulated yet, 1 when the row still has no key.
__device__ __forceinline__ float ref_advance(RowState& st, float ref_new, float c) {
  const float ninf = -__builtin_inff();
  const bool none_yet = st.ref == ninf, no_key = ref_new == ninf;
  const float arg = (none_yet || no_key) ? 0.0f : c * (st.ref - ref_new);
  float alpha = __builtin_amdgcn_exp2f(arg);
  alpha = none_yet ? 0.0f : alpha;
  st.ref = ref_new;
  return alpha;
}

template <int X, bool FB_AUTO>
__device__ __forceinline__ float row_state_update(RowState& st, float blk_max, float c, float tau) {
  row_max_update(st, blk_max);
  return ref_advance(st, block_ref<X, FB_AUTO>(st, c, tau), c);
}

// -c * ref, with a row that has no key yet mapped to 0 (its logits are all -inf,
// so every exponential is exactly 0 either way)
__device__ __forceinline__ float neg_c_ref(const RowState& st, float c) {
  return st.ref == -__builtin_inff() ? 0.0f : -c * st.ref;
}

}  // namespace tos
