// attn_fwd_f32_slab.hpp -- fp32 forward for problems too small to fill the GPU
// with 128-row workgroups (a single head of a few hundred rows, say), where the
// time of a launch is its latency: memory latency, the chain of dependent
// matrix instructions of one wave, and the merge.
//
// A workgroup takes a slab of 16 query rows of one head and a share 1/DS of
// the head dim of O.  Its 4 waves (one per SIMD) cut the slab's keys into
// contiguous ranges of 16-key chunks; each wave runs the tensorized online
// softmax over its own range (FlashAttention-T, section A2, "surrogate
// maximum": with X = 16 the reference is the largest running maximum of the
// slab's 16 rows, with X = 1 the row's own), and the workgroup merges the waves'
// partial results exactly through LDS:
//   m = max_w m_w,  l = sum_w 2^{c (m_w - m)} l_w,  O = sum_w 2^{c (m_w - m)} O_w / l,
// the rescale by exp(m_old - m_new) that the online softmax applies between
// consecutive key blocks (section A3, Fig 2(a)), here between key ranges.  With
// DS > 1 the DS workgroups of a slab each compute the whole of S = Q K^T (and
// the same P~) and their own columns of O: the launcher picks DS only when the
// DS-fold grid still fits the compute units, so the repeated S work takes
// compute units that would otherwise idle, and each one's chain of P~V
// instructions, V reads and merge shrink DS-fold.  One 128-row head of d = 64
// runs on 32 compute units instead of one.
//
// v_mfma_f32_16x16x4_f32 layout: A (16x4) lane L holds A[L%16][L/16]; B (4x16)
// lane L holds B[L/16][L%16]; the accumulator (16x16) lane L holds
// D[4 (L/16) + r][L%16], r = 0..3.  With g = L/16:
//  - S^T = K Q^T: step s contracts head dim (D/4) g + s for lane group g (any
//    assignment of the head dims to steps gives the same sum), so a lane's K
//    and Q operands are D/4 contiguous floats of one row, read as float4;
//  - O^T += V^T P~^T: P~^T is S^T's accumulator as it stands, step r
//    contracting key 4 g + r of the chunk; row i of output tile dt is head dim
//    DH h + DT i + dt of the workgroup's share h (DH = D/DS columns, DT = DH/16
//    tiles), so a lane's V operands for step r are DT contiguous floats of one
//    row, and its accumulators hold DT contiguous floats of its query per r.
#pragma once
#include "attn_fwd_kernels.hpp"

namespace tos {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSlabWaves = 4;   // the merge reads the waves' m and l as one float4
constexpr int kSlabThreads = 64 * kSlabWaves;
constexpr int kSlabRows = 16;    // query rows of a workgroup
constexpr int kSlabChunk = 16;   // keys per step of a wave

// combined over the four lane groups L, L^16, L^32, L^48 (one query's lanes)
template <typename Op>
__device__ __forceinline__ float group4_reduce(float x, Op op) {
  x = pair_reduce(x, op);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct AddOp { __device__ float operator()(float a, float b) const { return a + b; } };

template <int D, bool CAUSAL, int X, int DS>
__global__ __launch_bounds__(kSlabThreads, 1) void attn_fwd_f32_slab(FwdArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(X == 1 || X == 16, "tile rows: one query (X = 1) or the slab (X = 16)");
  static_assert(DS == 1 || DS == 2 || DS == 4, "head-dim shares");
  static_assert(kSlabWaves == 4, "the merge takes the waves' m and l as one float4");
  constexpr int QK = D / 4;      // floats of a lane's K or Q row segment
  constexpr int DH = D / DS;     // columns of O of this workgroup
  constexpr int DT = DH / 16;    // output tiles; V floats of a lane per key
  constexpr int VW = DT < 4 ? DT : 4;   // V floats per load
  typedef float fv __attribute__((ext_vector_type(VW)));
  constexpr int OS = DH + 4;     // LDS row stride of a partial O
  __shared__ __attribute__((aligned(16))) float o_part[kSlabWaves][kSlabRows * OS];
  // per query: the waves' m, then their l (one 16-byte read each in the merge)
  __shared__ __attribute__((aligned(16))) float ml_part[kSlabRows][2][kSlabWaves];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 15, g = lane >> 4;
  const int N = a.N;
  const int nslab = (N + kSlabRows - 1) / kSlabRows;
  // the DS shares of a slab are consecutive workgroups; causal: the slabs
  // with the most keys go first
  const int hh = (int)(blockIdx.x % DS);
  const unsigned bid = blockIdx.x / DS;
  const int bh = (int)(bid % (unsigned)a.BH);
  const int sl = CAUSAL ? nslab - 1 - (int)(bid / (unsigned)a.BH) : (int)(bid / (unsigned)a.BH);
  const int q0 = sl * kSlabRows;
  const int qrow = q0 + lq;
  const size_t head = (size_t)bh * N * D;
  const float* Q = (const float*)a.q + head;
  const float* K = (const float*)a.k + head;
  const float* V = (const float*)a.v + head;

  // the slab's keys, and this wave's chunks of them
  const int kend = CAUSAL ? min(q0 + kSlabRows, N) : N;
  const int nch = (kend + kSlabChunk - 1) / kSlabChunk;
  const int cb = w * nch / kSlabWaves, ce = (w + 1) * nch / kSlabWaves;
  const int klim = CAUSAL ? min(qrow + 1, N) : N;   // keys this lane's query sees

  f32x4 qf[QK / 4];
#pragma unroll
  for (int i = 0; i < QK / 4; ++i)
    qf[i] = qrow < N ? *(const f32x4*)(Q + (size_t)qrow * D + QK * g + 4 * i) : f32x4{};

  auto load_k = [&](int j, f32x4 (&kr)[QK / 4]) {
    const int key = j * kSlabChunk + lq;
#pragma unroll
    for (int i = 0; i < QK / 4; ++i)
      kr[i] = key < N ? *(const f32x4*)(K + (size_t)key * D + QK * g + 4 * i) : f32x4{};
  };
  auto load_v = [&](int j, fv (&vr)[4][DT / VW]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = j * kSlabChunk + 4 * g + r;
#pragma unroll
      for (int i = 0; i < DT / VW; ++i)
        vr[r][i] = key < N ? *(const fv*)(V + (size_t)key * D + DH * hh + DT * lq + VW * i) : fv{};
    }
  };

  const float c = a.c, ninf = -__builtin_inff();
  float m_run = ninf;   // running maximum: the query's (X = 1) or the slab's (X = 16)
  float lsum = 0.0f;    // this lane's share of the query's row sum
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{};

  f32x4 kc[QK / 4], kn[QK / 4];
  fv vc[4][DT / VW], vn[4][DT / VW];
  if (cb < ce) {
    load_k(cb, kc);
    load_v(cb, vc);
  }
  for (int j = cb; j < ce; ++j) {
    if (j + 1 < ce) {   // the next chunk's loads overlap this chunk's products
      load_k(j + 1, kn);
      load_v(j + 1, vn);
    }
    // S^T = K Q^T, the even and the odd steps in two chains
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < QK; s += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[s / 4][s % 4], qf[s / 4][s % 4], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[s / 4][s % 4 + 1], qf[s / 4][s % 4 + 1], s1, 0, 0, 0);
    }
    f32x4 sv = s0 + s1;
    const int kbase = j * kSlabChunk + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kbase + r >= klim) sv[r] = ninf;
    // the block's maximum of the query, then of the tile
    float mb = fmax_raw(fmax_raw(sv[0], sv[1]), fmax_raw(sv[2], sv[3]));
    mb = group4_reduce(mb, MaxOp());
    if constexpr (X == 16) mb = row16_reduce(mb, MaxOp());
    const float m_new = fmax_raw(m_run, mb);
    // alpha = 2^{c (m_old - m_new)}: 0 before the first key, 1 while there is none
    const float alpha = m_new == ninf ? 1.0f : __builtin_amdgcn_exp2f(c * (m_run - m_new));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      lsum *= alpha;
    }
    m_run = m_new;
    const float nb = m_new == ninf ? 0.0f : -c * m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, nb));
      lsum += sv[r];
    }
    // O^T += V^T P~^T
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vc[r][dt / VW][dt % VW], sv[r], oacc[dt], 0, 0, 0);
    if (j + 1 < ce) {
#pragma unroll
      for (int i = 0; i < QK / 4; ++i) kc[i] = kn[i];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < DT / VW; ++i) vc[r][i] = vn[r][i];
    }
  }

  // this wave's partial result: m, l and O of each query (a wave without
  // chunks leaves m = -inf, l = 0, O = 0, which the merge weighs by 0)
  const float l = group4_reduce(lsum, AddOp());
  if (lane < kSlabRows) {
    ml_part[lq][0][w] = m_run;
    ml_part[lq][1][w] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < DT / VW; ++i) {
      fv t;
#pragma unroll
      for (int u = 0; u < VW; ++u) t[u] = oacc[VW * i + u][r];
      *(fv*)(&o_part[w][lq * OS + DT * (4 * g + r) + VW * i]) = t;
    }
  __syncthreads();

  // merge: each thread a float4 of the workgroup's columns of the slab's O,
  // stored past the caches (nothing reads it again in this launch)
  constexpr int NV = kSlabRows * DH / 4;
  float* O = (float*)a.o + head + DH * hh;
#pragma unroll
  for (int u = tid; u < NV; u += kSlabThreads) {
    const int q = u / (DH / 4), d4 = 4 * (u % (DH / 4));
    const int row = q0 + q;
    if (row >= N) continue;
    const f32x4 mw = *(const f32x4*)&ml_part[q][0][0], lw = *(const f32x4*)&ml_part[q][1][0];
    const float M = fmax_raw(fmax_raw(mw[0], mw[1]), fmax_raw(mw[2], mw[3]));
    float L = 0.0f;
    f32x4 acc = {};
#pragma unroll
    for (int v = 0; v < kSlabWaves; ++v) {
      const float e = mw[v] == ninf ? 0.0f : __builtin_amdgcn_exp2f(c * (mw[v] - M));
      L += e * lw[v];
      acc += e * *(const f32x4*)(&o_part[v][q * OS + d4]);
    }
    const float inv = L > 0.0f ? a.o_scale / L : 0.0f;
    __builtin_nontemporal_store(acc * inv, (f32x4*)(O + (size_t)row * D + d4));
    if (a.lse != nullptr && hh == 0 && d4 == 0)
      a.lse[(size_t)bh * N + row] = L > 0.0f ? a.lse_scale * M + __logf(L) : ninf;
  }
}

}  // namespace tos
