// attn_fwd_kernels.hpp -- fused attention forward kernels for gfx950 (MI355X).
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns
// 32 query rows.  Keys stream through LDS in blocks of 64 (double-buffered: the
// global loads of block j+1 are in flight while block j is computed).  Per key
// block each wave runs the fused-attention iteration of FlashAttention-T
// (section A3, Fig 2(a)) with the tensorized online softmax (section A2,
// Algorithm 1):
//   S^T = K_j Q^T                          (MFMA; Q held in registers)
//   tile max m^ -> uniform alpha, O *= alpha, l *= alpha    (steps 1-3)
//   P~ = exp2(c*S - c*m^)                  (steps 4-6: one FMA + v_exp_f32)
//   l += rowsum(P~)                        (step 7: VALU dot products of packed
//                                           P~ pairs with (1,1), or an MFMA with
//                                           an all-ones operand)
//   O^T += V_j^T P~^T                      (MFMA)
// Computing the transposed products keeps every per-row quantity in one lane
// pair: the 32x32 MFMA accumulator gives lane L the column L mod 32 = one query.
// The P~ operand of the second product is read straight out of the first
// product's accumulator registers: the key order inside each 16-key step is
// permuted to match, and V's operand is read from LDS in the same permuted
// order with the transposing LDS read (ds_read_b64_tr_b16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "softmax_tile.hpp"

namespace tos {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;            // batch * heads
  int N;             // sequence length
  int nqb;           // query blocks per head = ceil(N / 128)
  float c;           // scale * log2(e) (fp8: times the q and k descales)
  float lse_scale;   // scale (fp8: times the q and k descales)
  float o_scale;     // multiplies O at the end (fp8: the v descale)
  float tau;         // fallback threshold, log2 units
  int* fallback_tiles;   // per-row tile counter, or nullptr
  int count_x;       // > 0: count the X-row tiles of this size as per-row (FORCE)
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
constexpr int kBc = 64;            // keys per block

__device__ __forceinline__ void block_coords(const FwdArgs& a, bool causal, int& bh, int& q0) {
  // causal: the heaviest query blocks (most keys) go first; consecutive block
  // ids walk the heads, so with BH a multiple of 8 every workgroup of a head
  // lands on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
  const int bid = blockIdx.x;
  bh = bid % a.BH;
  const int qb = causal ? (a.nqb - 1 - bid / a.BH) : bid / a.BH;
  q0 = qb * kBr;
}

// Tile counter: once per tile that ran with per-row maxima.
template <int X, bool FB_AUTO>
__device__ __forceinline__ void count_tiles(const FwdArgs& a, const RowState& st, int lane,
                                            int qrow) {
  if (a.fallback_tiles == nullptr || lane >= 32 || qrow >= a.N) return;
  if constexpr (FB_AUTO) {
    if (st.per_row && (lane % X) == 0) atomicAdd(a.fallback_tiles, 1);
  } else {
    if (a.count_x > 0 && (qrow % a.count_x) == 0) atomicAdd(a.fallback_tiles, 1);
  }
}

// ---------------------------------------------------------------------------
// bf16: v_mfma_f32_32x32x16_bf16 for both products.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int X, bool ROWSUM_MFMA, bool FB_AUTO>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16(FwdArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D + 8;    // K row stride in LDS (elements): rows 4 banks apart
  constexpr int VS = D + 32;   // V row stride: transposing reads hit 4 rows x 32 B
  constexpr int CH = kBc * D / 8 / kThreads;   // 16-byte chunks per thread per tensor
  constexpr int NKK = D / 16;  // k-steps of S^T = K Q^T
  constexpr int NMT = D / 32;  // 32-row M tiles of O^T
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * kBc * KS + 2 * kBc * VS];
  __bf16* kl = smem;
  __bf16* vl = smem + 2 * kBc * KS;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  int bh, q0;
  block_coords(a, CAUSAL, bh, q0);
  const int N = a.N;
  const int qrow = q0 + 32 * w + ln;
  const bool qvalid = qrow < N;
  const size_t head = (size_t)bh * N * D;
  const __bf16* Q = (const __bf16*)a.q + head;
  const __bf16* K = (const __bf16*)a.k + head;
  const __bf16* V = (const __bf16*)a.v + head;

  // key blocks: all of them, or (causal) up to the workgroup's last query
  const int nblk = (N + kBc - 1) / kBc;
  const int qlast_wg = min(q0 + kBr, N) - 1;
  const int jend = CAUSAL ? qlast_wg / kBc + 1 : nblk;
  const int wq0 = q0 + 32 * w;                       // first query of the wave
  const int wqlast = min(wq0 + 31, N - 1);
  const int jend_w = (wq0 >= N) ? 0 : (CAUSAL ? wqlast / kBc + 1 : nblk);
  // keys this lane may see: [0, klim)
  const int klim = qvalid ? (CAUSAL ? qrow + 1 : N) : 0;

  // Q^T operand: lane (query ln, half hf) holds Q[qrow][16 kk + 8 hf + 0..7]
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (qvalid)
      qf[kk] = *(const bf16x8*)(Q + (size_t)qrow * D + 16 * kk + 8 * hf);
    else
      qf[kk] = bf16x8{};
  }

  u32x4 kreg[CH], vreg[CH];
  auto gload = [&](int j) {
    const int kb = j * kBc;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + kThreads * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      if (kb + row < N) {
        kreg[i] = *(const u32x4*)(K + (size_t)(kb + row) * D + col);
        vreg[i] = *(const u32x4*)(V + (size_t)(kb + row) * D + col);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};   // keys past N: zero K (masked) and zero V
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + kThreads * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(u32x4*)(kl + buf * kBc * KS + row * KS + col) = kreg[i];
      *(u32x4*)(vl + buf * kBc * VS + row * VS + col) = vreg[i];
    }
  };

  RowState st;
  row_state_init(st, X == 1);
  const float c = a.c, tau = a.tau;
  f32x16 oacc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) oacc[mt] = f32x16{};
  float lsum = 0.0f;    // row sum of the rounded P~ (VALU; this lane's keys only)
  f32x16 lacc = {};     // the same on the MFMA (every register holds the full sum)
  float lexact = 0.0f;  // row sum of the unrounded P~ (this lane's keys only)
  bf16x8 ones;
#pragma unroll
  for (int t = 0; t < 8; ++t) ones[t] = (__bf16)1.0f;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  if (jend > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int j = 0; j < jend; ++j) {
    const int buf = j & 1;
    if (j + 1 < jend) gload(j + 1);
    if (j < jend_w) {
      const __bf16* kt = kl + buf * kBc * KS;
      const __bf16* vt = vl + buf * kBc * VS;
      // ---- S^T = K_j Q^T: two 32-key tiles
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a0 = *(const bf16x8*)(kt + ln * KS + 16 * kk + 8 * hf);
        const bf16x8 a1 = *(const bf16x8*)(kt + (32 + ln) * KS + 16 * kk + 8 * hf);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s1, 0, 0, 0);
      }
      // ---- mask: key index of register r of tile t is kb + 32t + 8(r/4) + 4hf + r%4
      const int kb = j * kBc;
      const bool need_mask = (kb + kBc > N) || (wq0 + 32 > N) || (CAUSAL && kb + kBc > wq0 + 1);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r / 4) + 4 * hf + (r % 4);
          if (key >= klim) s0[r] = -__builtin_inff();
          if (key + 32 >= klim) s1[r] = -__builtin_inff();
        }
      }
      // ---- Algorithm 1 step 1 and the reference update (steps 2-3)
      float bm = s0[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmax_raw(bm, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) bm = fmax_raw(bm, s1[r]);
      const float alpha = row_state_update<X, FB_AUTO>(st, bm, c, tau);
      // uniform over the tile; the whole wave skips the rescale when no row's
      // reference moved (alpha == 1 everywhere)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) oacc[mt] *= alpha;
        if constexpr (ROWSUM_MFMA)
          lacc *= alpha;
        else
          lsum *= alpha;
        lexact *= alpha;
      }
      // ---- steps 4-6: P~ = exp2(c*S - c*ref), packed to bf16 as the B operand
      const float nb = neg_c_ref(st, c);
      bf16x8 pk[4];
      float pe0 = 0.0f, pe1 = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, nb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, nb));
        pe0 += p0;
        pe1 += p1;
        pk[r / 8][r % 8] = (__bf16)p0;
        pk[2 + r / 8][r % 8] = (__bf16)p1;
      }
      // two row sums (step 7): the unrounded one gives lse; the one over the
      // rounded P~ the P~V product consumes normalises O, so O / l stays a
      // weighted average of V rows (bf16 rounding of P~ then cancels to first
      // order instead of adding to the error of O)
      lexact += pe0 + pe1;
      if constexpr (!ROWSUM_MFMA) {
        // on the vector unit: dot products of each packed pair with (1, 1)
        float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ps[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 0, 1), ones2, ps[0], false);
          ps[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 2, 3), ones2, ps[1], false);
          ps[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 4, 5), ones2, ps[2], false);
          ps[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 6, 7), ones2, ps[3], false);
        }
        lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      }
      // ---- O^T += V_j^T P~^T, 16 keys per step.  Step s, slot t of lane half h
      // is key 16s + 8(t/4) + 4h + t%4 (the accumulator order above); the
      // transposing read gives lane (16-lane group G, index i) the V row
      // 16s + 4(G/2) + i/4 (+8 for slots 4..7) at columns 16(G%2) + 4(i%4).
      const int G = lane >> 4, gi = lane & 15;
      const int vrow = 4 * (G >> 1) + (gi >> 2);
      const int vcol = 16 * (G & 1) + 4 * (gi & 3);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const __bf16* p = vt + (16 * s + vrow) * VS + 32 * mt + vcol;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(p));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(p + 8 * VS));
          const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 av = __builtin_bit_cast(bf16x8, both);
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[s], oacc[mt], 0, 0, 0);
        }
        if constexpr (ROWSUM_MFMA)   // step 7 on the matrix unit: ones x P~^T
          lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pk[s], lacc, 0, 0, 0);
      }
    }
    if (j + 1 < jend) lstore((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: l, O / l, lse (reading R-7: lse = scale*ref + ln l)
  float l;
  if constexpr (ROWSUM_MFMA)
    l = lacc[0];
  else
    l = pair_reduce(lsum, [](float x, float y) { return x + y; });
  const float le = pair_reduce(lexact, [](float x, float y) { return x + y; });
  const float inv = l > 0.0f ? a.o_scale / l : 0.0f;
  if (qvalid) {
    __bf16* O = (__bf16*)a.o + head + (size_t)qrow * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int t = 0; t < 4; ++t) ov[t] = (__bf16)(oacc[mt][4 * g + t] * inv);
        *(bf16x4*)(O + 32 * mt + 8 * g + 4 * hf) = ov;
      }
    }
    if (a.lse != nullptr && hf == 0)
      a.lse[(size_t)bh * N + qrow] =
          le > 0.0f ? a.lse_scale * st.ref + __logf(le) : -__builtin_inff();
  }
  count_tiles<X, FB_AUTO>(a, st, lane, qrow);
}

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32 for both products, P~ kept in fp32.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int X, bool FB_AUTO>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32(FwdArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D + 1;   // odd stride: a column read hits 32 distinct banks
  constexpr int VS = D;       // row reads of 32 consecutive floats
  constexpr int CH = kBc * D / 4 / kThreads;   // 16-byte chunks per thread per tensor
  constexpr int NMT = D / 32;
  __shared__ float kl[kBc * KS];
  __shared__ __attribute__((aligned(16))) float vl[kBc * VS];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  int bh, q0;
  block_coords(a, CAUSAL, bh, q0);
  const int N = a.N;
  const int qrow = q0 + 32 * w + ln;
  const bool qvalid = qrow < N;
  const size_t head = (size_t)bh * N * D;
  const float* Q = (const float*)a.q + head;
  const float* K = (const float*)a.k + head;
  const float* V = (const float*)a.v + head;
  const int nblk = (N + kBc - 1) / kBc;
  const int qlast_wg = min(q0 + kBr, N) - 1;
  const int jend = CAUSAL ? qlast_wg / kBc + 1 : nblk;
  const int wq0 = q0 + 32 * w;
  const int wqlast = min(wq0 + 31, N - 1);
  const int jend_w = (wq0 >= N) ? 0 : (CAUSAL ? wqlast / kBc + 1 : nblk);
  const int klim = qvalid ? (CAUSAL ? qrow + 1 : N) : 0;

  // Q^T operand: lane (query ln, half hf) holds Q[qrow][2 kk + hf]
  float qf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qvalid ? Q[(size_t)qrow * D + 2 * kk + hf] : 0.0f;

  RowState st;
  row_state_init(st, X == 1);
  const float c = a.c, tau = a.tau;
  f32x16 oacc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) oacc[mt] = f32x16{};
  float lsum = 0.0f;

  for (int j = 0; j < jend; ++j) {
    const int kb = j * kBc;
    __syncthreads();   // previous block fully consumed
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int cidx = tid + kThreads * i, row = cidx / (D / 4), col = (cidx % (D / 4)) * 4;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (kb + row < N) {
        kv = *(const u32x4*)(K + (size_t)(kb + row) * D + col);
        vv = *(const u32x4*)(V + (size_t)(kb + row) * D + col);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) kl[row * KS + col + t] = __uint_as_float(kv[t]);
      *(u32x4*)(vl + row * VS + col) = vv;
    }
    __syncthreads();
    if (j >= jend_w) continue;
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[ln * KS + 2 * kk + hf], qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[(32 + ln) * KS + 2 * kk + hf], qf[kk], s1, 0, 0, 0);
    }
    const bool need_mask = (kb + kBc > N) || (wq0 + 32 > N) || (CAUSAL && kb + kBc > wq0 + 1);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 8 * (r / 4) + 4 * hf + (r % 4);
        if (key >= klim) s0[r] = -__builtin_inff();
        if (key + 32 >= klim) s1[r] = -__builtin_inff();
      }
    }
    float bm = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bm = fmax_raw(bm, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) bm = fmax_raw(bm, s1[r]);
    const float alpha = row_state_update<X, FB_AUTO>(st, bm, c, tau);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) oacc[mt] *= alpha;
      lsum *= alpha;
    }
    const float nb = neg_c_ref(st, c);
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, nb));
      s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, nb));
      ps += s0[r] + s1[r];
    }
    lsum += ps;
    // O^T += V^T P~^T, one key per lane half per step: step (tile t, reg r)
    // contracts key 32t + 8(r/4) + 4h + r%4 for lane half h
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key0 = 8 * (r / 4) + 4 * hf + (r % 4);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[key0 * VS + 32 * mt + ln], s0[r], oacc[mt], 0, 0, 0);
        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[(32 + key0) * VS + 32 * mt + ln], s1[r], oacc[mt], 0, 0, 0);
      }
    }
  }

  const float l = pair_reduce(lsum, [](float x, float y) { return x + y; });
  const float inv = l > 0.0f ? a.o_scale / l : 0.0f;
  if (qvalid) {
    float* O = (float*)a.o + head + (size_t)qrow * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 ov = make_float4(oacc[mt][4 * g] * inv, oacc[mt][4 * g + 1] * inv,
                                oacc[mt][4 * g + 2] * inv, oacc[mt][4 * g + 3] * inv);
        *(float4*)(O + 32 * mt + 8 * g + 4 * hf) = ov;
      }
    }
    if (a.lse != nullptr && hf == 0)
      a.lse[(size_t)bh * N + qrow] =
          l > 0.0f ? a.lse_scale * st.ref + __logf(l) : -__builtin_inff();
  }
  count_tiles<X, FB_AUTO>(a, st, lane, qrow);
}

}  // namespace tos
