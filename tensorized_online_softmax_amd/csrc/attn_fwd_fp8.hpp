// attn_fwd_fp8.hpp -- the fused attention forward kernel for OCP fp8 e4m3
// inputs on gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4 for both products).
//
// Same method, workgroup shape and persistent item loop as the 16-bit kernel
// (8 waves = 256 query rows, 64-key blocks streamed through LDS rings by
// direct-to-LDS loads, O stored through LDS as whole rows, the tensorized
// online softmax of FlashAttention-T, section A2, Algorithm 1, with the
// optional per-row fallback of "numerical stability guarantees").
// What differs for fp8:
//   * Q, K, V are e4m3 codes with per-tensor fp32 descales; the logit scale
//     c = scale * log2(e) * q_descale * k_descale, and O is multiplied by
//     v_descale at the end.
//   * One MFMA contracts 64 values: S^T = K Q^T takes 2 k-steps per 32-key
//     tile, O^T += V^T P~^T one instruction per 32-row M tile and 64 keys.
//   * P~ enters the second product as e4m3, after a 2^8 pre-scale folded
//     into the exponent (P~ <= 1 becomes <= 256 < 448, and the e4m3 normal
//     range then starts at P~ = 2^-14).  The fallback threshold tau (default
//     12) keeps every row's largest term at or above 2^-12.
//   * As two e4m3 terms: hi = e4m3(2^8 P~) and lo = e4m3(2^8 P~ - hi), each
//     with its own MFMA.  One e4m3 rounding (3 mantissa bits) alone moves O
//     by up to 6e-2 and more on rows that average two or three keys (the
//     oracle's model of it shows this on the stress construction); hi + lo
//     is within 2^-8 of 2^8 P~.  Values below the e4m3 range still flush to
//     zero in both terms, so the underflow the fallback guards against is
//     unchanged.  The kernel is bound by its vector work, so the extra matrix
//     instructions cost little.
//   * The row sum that normalises O is the sum of hi + lo that the product
//     consumes, taken on the matrix unit (an all-ones operand against each
//     term) for the blocks of a wave's edge steps, and the unrounded fp32 sum
//     for those of its steady steps (see steady_step); the unrounded fp32 sum
//     of every block gives lse.
//
// Operand layouts (32x32x64 e4m3, measured on gfx950): slot t of lane half h
// of the A operand meets slot t of lane half h of the B operand.  So, as in
// the bf16 kernel, the key order of the P~V contraction is the accumulator
// order of S^T: slot 16u + r of half h is key 32u + 8(r/4) + 4h + r%4 of the
// block (tile u, register r), and V's operand is fetched in that order by
// ds_read_b64_tr_b8 (per 16-lane group, lane j's byte t comes from the
// address of lane 2t + j/8, at byte offset j%8 of it).
//
// LDS rows are d bytes, 16-byte chunks XOR-swizzled (f8_kswz, f8_vswz):
//   d = 128: K chunk c of row r at c ^ (r & 7), V at c ^ ((r >> 1) & 7)
//   d = 64:  K chunk c of row r at c ^ ((r >> 2) & 3), V at c ^ (2 ((r >> 3) & 1))
// which keeps the K operand reads (16 rows x 16 bytes per 16 lanes) and the
// transposing V reads (16 rows x 32 bytes per instruction) conflict-free.
// At d = 128 every wave loads 1 KiB of K and 1 KiB of V per step; at d = 64 a
// block is 4 KiB, so waves 0-3 load K and waves 4-7 load V, 1 KiB each.
#pragma once
#include "attn_fwd_kernels.hpp"

namespace tos {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kF8PreScaleLog2 = 8;   // P~ * 2^8 is stored as e4m3

template <int D> __device__ __forceinline__ int f8_kswz(int r, int c) {
  return D == 128 ? (c ^ (r & 7)) : (c ^ ((r >> 2) & 3));
}
template <int D> __device__ __forceinline__ int f8_vswz(int r, int c) {
  return D == 128 ? (c ^ ((r >> 1) & 7)) : (c ^ (2 * ((r >> 3) & 1)));
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = e4m3 for both operands, unit (2^0) block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int D, bool CAUSAL, int X, bool FB_AUTO>
__global__ __launch_bounds__(kPThreads, 1) void attn_fwd_fp8(FwdArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int RB = D;                       // bytes per K or V row
  constexpr int CPR = RB / 16;                // 16-byte chunks per row
  constexpr int BLK = kBc * RB;               // bytes per key block (8 or 4 KiB)
  constexpr bool SPLIT = D == 64;             // waves 0-3 load K, 4-7 load V
  constexpr int NV_STEP = SPLIT ? 1 : 2;      // 1 KiB loads a wave issues per step
  constexpr int NKK = D / 64;                 // k-steps of S^T = K Q^T
  constexpr int NQK = 2 * NKK;                // QK matrix instructions per block
  constexpr int NMT = D / 32;                 // 32-row M tiles of O^T
  // Past the rings, 8 x 32 rows of bf16 O staging (one area per wave), as in
  // the 16-bit kernel: O leaves through LDS as whole rows.
  constexpr int ORB = 2 * D;                  // bytes per O row (bf16)
  constexpr int SB = 32 * ORB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kRing * BLK + kPWaves * SB];
  char* vring = smem;

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Persistent workgroups over items, as in the 16-bit kernel (item_of).
  const int N = a.N;
  const int nblk = (N + kBc - 1) / kBc;
  const int nitems = a.BH * a.nqb;
  const int nwg = gridDim.x, gid = blockIdx.x;
  auto item_jend = [&](int q0_) { return CAUSAL ? (min(q0_ + kPBr, N) - 1) / kBc + 1 : nblk; };

  int bh = 0, q0 = 0, qrow = 0, jend = 0, jend_w = 0, klim = 0;
  bool qvalid = false;
  size_t head = 0;
  u32x4 kdesc = {}, vdesc = {};
  auto set_item = [&](int it) {
    int qb;
    item_coords(a, CAUSAL, it, bh, qb);
    q0 = qb * kPBr;
    qrow = q0 + 32 * w + ln;
    qvalid = qrow < N;
    head = (size_t)bh * N * D;
    kdesc = buffer_desc((const unsigned char*)a.k + head, (unsigned)N * RB);
    vdesc = buffer_desc((const unsigned char*)a.v + head, (unsigned)N * RB);
    jend = item_jend(q0);
    const int wq0 = q0 + 32 * w;
    jend_w = (wq0 >= N) ? 0 : (CAUSAL ? min(wq0 + 31, N - 1) / kBc + 1 : nblk);
    klim = qvalid ? (CAUSAL ? qrow + 1 : N) : 0;
  };
  // the next item's first K and V blocks ride on this item's last steps when
  // this item's block count is a multiple of the ring size; its Q is loaded
  // in this item's last step
  bool pref_next = false;
  int jend_n = 0, qrow_n = 0;
  bool qvalid_n = false;
  size_t head_n = 0;
  u32x4 kdesc_n = {}, vdesc_n = {};
  auto set_next = [&](int it) {
    pref_next = it < nitems && jend % kRing == 0;
    if (pref_next) {
      int bh_n, qb_n;
      item_coords(a, CAUSAL, it, bh_n, qb_n);
      head_n = (size_t)bh_n * N * D;
      kdesc_n = buffer_desc((const unsigned char*)a.k + head_n, (unsigned)N * RB);
      vdesc_n = buffer_desc((const unsigned char*)a.v + head_n, (unsigned)N * RB);
      jend_n = item_jend(qb_n * kPBr);
      qrow_n = qb_n * kPBr + 32 * w + ln;
      qvalid_n = qrow_n < N;
    }
  };

  // Q^T operand of k-step kk: lane (query ln, half hf) holds Q[qrow][64 kk + 32 hf + 0..31]
  i32x8 qf[NKK];
  auto load_q = [&](size_t head_, int qrow_, bool qvalid_) {
    const unsigned char* Q = (const unsigned char*)a.q + head_;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qvalid_) {
        const u32x4* src = (const u32x4*)(Q + (size_t)qrow_ * D + 64 * kk + 32 * hf);
        const u32x4 lo = src[0], hi = src[1];
        qf[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        qf[kk] = i32x8{};
      }
    }
  };

  // direct-to-LDS loads: lane L of the wave with share s (s = w, or w mod 4
  // when the waves split K and V) fills bytes [1024 s + 16 L, +16) of the slot
  // = row r = (1024 s + 16 L) / RB, chunk position p, fetching the chunk that
  // the swizzle puts there
  const int ws = SPLIT ? (w & 3) : w;
  unsigned kgoff[1], vgoff[1];
  {
    const int r = (1024 * ws + 16 * lane) / RB, p = lane % CPR;
    kgoff[0] = (unsigned)(r * RB + 16 * f8_kswz<D>(r, p));
    vgoff[0] = (unsigned)(r * RB + 16 * f8_vswz<D>(r, p));
  }
  const unsigned lds0 = (unsigned)(unsigned long long)(__attribute__((address_space(3))) char*)smem;
  const unsigned vdst = lds0 + (unsigned)ws * 1024, kdst = vdst + kRing * BLK;
  const bool loads_k = !SPLIT || w < 4, loads_v = !SPLIT || w >= 4;   // wave-uniform
  // block j of the item's K (V), zeros past its end; with XING the blocks past
  // the end are the next item's first ones when those are prefetched
  auto ring_desc = [&](const u32x4& cur, const u32x4& nxt, int j) -> u32x4 {
    return select_desc(pref_next & (j >= jend), block_desc(nxt, j - jend, jend_n, BLK),
                       block_desc(cur, j, jend, BLK));
  };
  auto load_k = [&](int j, auto XING) {
    if (!loads_k) return;
    if constexpr (decltype(XING)::value)
      dma_block<1>(ring_desc(kdesc, kdesc_n, j), kdst + (j % kRing) * BLK, kgoff);
    else
      dma_block<1>(block_desc(kdesc, j, jend, BLK), kdst + (j % kRing) * BLK, kgoff);
  };
  auto load_v = [&](int j, auto XING) {
    if (!loads_v) return;
    if constexpr (decltype(XING)::value)
      dma_block<1>(ring_desc(vdesc, vdesc_n, j), vdst + (j % kRing) * BLK, vgoff);
    else
      dma_block<1>(block_desc(vdesc, j, jend, BLK), vdst + (j % kRing) * BLK, vgoff);
  };

  // K operand of tile u, k-step kk: lane (key ln, half hf) reads the 32 bytes
  // of chunks 4kk + 2hf, +1 of row 32u + ln (the swizzle depends on ln only
  // through bits that 32u does not touch)
  int koff[NKK][2];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[kk][e] = kRing * BLK + ln * RB + 16 * f8_kswz<D>(ln, 4 * kk + 2 * hf + e);
  // V operand of M tile mt, read c (0..3): lane L addresses row 16c + f(L) at
  // column 32 mt + g(L): f = 8(t/4) + 4h + t%4 with t = (L%16)/2, h = L/32;
  // g = 16((L/16)%2) + 8(L%2).  The swizzle of row 16c + f does not depend on c.
  int voff[NMT];
  {
    const int t = (lane % 16) / 2, f = 8 * (t / 4) + 4 * hf + t % 4;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      voff[mt] = f * RB + 16 * f8_vswz<D>(f, 2 * mt + (lane / 16) % 2) + 8 * (lane % 2);
  }

  RowState st;
  const float c = a.c, tau = a.tau;
  f32x16 oacc[NMT];
  float ledge;      // row sum of hi + lo of 2^8 P~ over the edge steps (from
                    // the matrix unit; both lanes of the pair hold it)
  float lsteady;    // row sum of the unrounded 2^8 P~ over the steady steps
                    // (this lane's keys only)
  float lexact;     // row sum of the unrounded 2^8 P~ (this lane's keys only)
  // pipeline registers: entering step j, S_j in S[0] and the hi and lo terms
  // of P~_{j-1} in PH[1], PL[1] (the steady steps alternate the two sets)
  f32x16 S[2][2];
  i32x8 PH[2], PL[2];
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0

  auto kread = [&](int slot, int u, int kk) -> i32x8 {
    const char* kt = smem + slot * BLK + u * 32 * RB;
    const u32x4 lo = *(const u32x4*)(kt + koff[kk][0]);
    const u32x4 hi = *(const u32x4*)(kt + koff[kk][1]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto vread = [&](int slot, int mt) -> i32x8 {
    const char* p = vring + slot * BLK + voff[mt];
    i32x8 r;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(p + cc * 16 * RB));
      r[2 * cc] = x[0];
      r[2 * cc + 1] = x[1];
    }
    return r;
  };
  // S^T = K_j Q^T into (s0, s1)
  auto qk = [&](int slot, f32x16& s0, f32x16& s1) {
    s0 = mfma_f8(kread(slot, 0, 0), qf[0], f32x16{});
    s1 = mfma_f8(kread(slot, 1, 0), qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < NKK; ++kk) {
      s0 = mfma_f8(kread(slot, 0, kk), qf[kk], s0);
      s1 = mfma_f8(kread(slot, 1, kk), qf[kk], s1);
    }
  };
  // O^T += V_j^T (hi + lo)^T
  auto pv = [&](int slot, const i32x8& hi, const i32x8& lo) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const i32x8 vop = vread(slot, mt);
      oacc[mt] = mfma_f8(vop, hi, oacc[mt]);
      oacc[mt] = mfma_f8(vop, lo, oacc[mt]);
    }
  };

  // ---- the softmax of one key block (Algorithm 1), in pieces
  // key of register r of tile u in block j: j*Bc + 32u + 8(r/4) + 4hf + r%4
  auto mask_block = [&](int j, f32x16& s0, f32x16& s1) {
    const int kb = j * kBc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + 8 * (r / 4) + 4 * hf + (r % 4);
      if (key >= klim) s0[r] = -__builtin_inff();
      if (key + 32 >= klim) s1[r] = -__builtin_inff();
    }
  };
  float m4[4];
  auto max_part = [&](int q, const f32x16& s0, const f32x16& s1) {
    const f32x16& sv = (q / 2) ? s1 : s0;
    const int r0 = 8 * (q % 2);
    float m = fmax_raw(sv[r0], sv[r0 + 1]);
#pragma unroll
    for (int r = r0 + 2; r < r0 + 8; r += 2) m = fmax3_raw(m, sv[r], sv[r + 1]);
    m4[q] = m;
  };
  float ref_new = 0.0f;
  auto max_combine = [&]() {
    float bm = fmax_raw(fmax3_raw(m4[0], m4[1], m4[2]), m4[3]);
    bm = qvalid ? bm : -__builtin_inff();
    row_max_update(st, bm);
  };
  auto tile_ref = [&]() {
    if constexpr (FB_AUTO && X > 1) {
      // a tile that went per-row stays so: once every tile of the wave has
      // (most tiles of data with spiky rows), the tile maximum and minimum
      // are not needed any more (a uniform branch)
      if (__builtin_amdgcn_ballot_w64(!st.per_row) == 0) {
        ref_new = st.m_run;
        return;
      }
    }
    ref_new = block_ref<X, FB_AUTO>(st, c, tau);
  };
  // alpha, and -c*ref + 8: the 2^8 pre-scale rides on the exponent
  auto advance = [&](float& alpha, float& nb) {
    alpha = ref_advance(st, ref_new, c);
    nb = neg_c_ref(st, c) + (float)kF8PreScaleLog2;
  };
  // steps 4-7 for registers r..r+3 of tile u (unit k: u = k / 4, r = 4 (k % 4)):
  // 2^8 P~ = exp2(c*S - c*ref + 8) as hi + lo e4m3 terms (operand dword 4u + r/4),
  // and the unrounded row sum
  // (in three stages, as in the 16-bit kernel, so that a steady step can put
  // them in different chunks: the FMAs, the exponentials, then the sum and
  // the hi / lo packing)
  float pe[2];
  float fz[8][4], fp[8][4];   // per unit: Z, then 2^8 P~ (registers, unrolled)
  auto unit_fma = [&](int k, const f32x16& s0, const f32x16& s1, float nb) {
    const int u = k / 4, r = 4 * (k % 4);
    const f32x16& sv = u ? s1 : s0;
#pragma unroll
    for (int e = 0; e < 4; ++e) fz[k][e] = __builtin_fmaf(sv[r + e], c, nb);
  };
  auto unit_exp = [&](int k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) fp[k][e] = __builtin_amdgcn_exp2f(fz[k][e]);
  };
  auto unit_sum_pack = [&](int k, i32x8& pk, i32x8& pl) {
    const int u = k / 4, r = 4 * (k % 4);
    const float* p = fp[k];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[u] += p[e];
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
    pk[4 * u + r / 4] = wd;
    const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false);
    const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
    int wl = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] - h01[0], p[1] - h01[1], 0, false);
    wl = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] - h23[0], p[3] - h23[1], wl, true);
    pl[4 * u + r / 4] = wl;
  };
  auto exp_unit = [&](int k, const f32x16& s0, const f32x16& s1, i32x8& pk, i32x8& pl, float nb) {
    unit_fma(k, s0, s1, nb);
    unit_exp(k);
    unit_sum_pack(k, pk, pl);
  };
  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) oacc[mt] *= alpha;
      ledge *= alpha;
    }
  };
  auto step_loads = [&](int j, auto XING) {
    load_k(j + kKAhead, XING);
    load_v(j + kVAhead, XING);
  };

  // Pipeline of key block b (as in the 16-bit kernel): S_b = K_b Q^T in step
  // b-1; its tile maximum, exponentials and row sums in step b, where O is
  // rescaled by alpha_b at the end; P~_b V_b in step b+1.  The last step
  // (j = jend) loads the next item's Q instead of K and V when the next item
  // is prefetched.
  auto edge_step = [&](int j) {
    if (pref_next && j == jend)
      load_q(head_n, qrow_n, qvalid_n);
    else
      step_loads(j, Int<1>());
    float alpha = 1.0f, nb = 0.0f;
    if (j < jend_w) {
      if (j == jend_w - 1) mask_block(j, S[0][0], S[0][1]);
#pragma unroll
      for (int q = 0; q < 4; ++q) max_part(q, S[0][0], S[0][1]);
      max_combine();
      tile_ref();
      advance(alpha, nb);
      pe[0] = pe[1] = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) exp_unit(k, S[0][0], S[0][1], PH[0], PL[0], nb);
      lexact = lexact * alpha + (pe[0] + pe[1]);
      lsteady *= alpha;
    }
    if (j + 1 < jend_w) qk((j + 1) % kRing, S[0][0], S[0][1]);
    if (j >= 1 && j <= jend_w) pv((j - 1) % kRing, PH[1], PL[1]);
    step_barrier<2 * NV_STEP>();
    if (j < jend_w) {
      rescale(alpha);
      // this block's rounded row sum (ones x (hi + lo)^T), after the rescale:
      // its terms are relative to the new reference already
      // (every register of the product holds the sum: one float carries it,
      // and the rescales multiply one float instead of sixteen)
      ledge += mfma_f8(ones, PL[0], mfma_f8(ones, PH[0], f32x16{}))[0];
    }
    PH[1] = PH[0];
    PL[1] = PL[0];
  };

  // Steady step j = 1 + 4g + u: j >= 1 and S_j is not the wave's last block.
  // One straight-line block of matrix-instruction chunks:
  //   A (4 chunks): S_{j+1} = K_{j+1} Q^T, each with a part of the tile-maximum
  //                 chain of S_j (parts 0-1 | 2-3 | combine + tile max | advance)
  //   B (8 chunks): O^T += V_{j-1}^T (hi + lo)^T, with the 8 exponential units
  //                 of S_j
  // The rounded row sum (ones x (hi + lo)^T on the matrix unit) is taken for
  // the blocks of the edge steps only (a wave's first and last key blocks,
  // which hold every key of a row that has few); a steady step adds the
  // unrounded sum of its block to O's normaliser instead (such a row has more
  // than 128 keys, over which the rounding of hi + lo averages out), which
  // saves two matrix instructions of 64 clocks per step.
  // Constant ring slots (four steps per loop iteration); S and P~ alternate
  // between the two register sets.
  auto steady_step = [&](auto U, int j, auto XING) {
    constexpr int u = decltype(U)::value;
    constexpr int cur = u & 1, nxt = cur ^ 1;
    constexpr int kslot = (u + 2) % kRing, vslot = u % kRing;   // K_{j+1}, V_{j-1}
    f32x16 &c0 = S[cur][0], &c1 = S[cur][1], &n0 = S[nxt][0], &n1 = S[nxt][1];
    step_loads(j, XING);
    float alpha = 1.0f, nb = 0.0f;
    pe[0] = pe[1] = 0.0f;
    // phase A at raised wave priority, phase B at the default (as in the
    // 16-bit kernel: of the two waves of a SIMD, the one behind issues first)
    __builtin_amdgcn_s_setprio(1);
    // phase A: QK g = 2 kk + t, operands read one instruction ahead
    i32x8 kop = kread(kslot, 0, 0);
#pragma unroll
    for (int g = 0; g < NQK; ++g) {
      const i32x8 av = kop;
      if (g + 1 < NQK) kop = kread(kslot, (g + 1) % 2, (g + 1) / 2);
      f32x16& acc = (g % 2) ? n1 : n0;
      acc = mfma_f8(av, qf[g / 2], g < 2 ? f32x16{} : acc);
      if constexpr (NQK == 4) {
        if (g == 0) { max_part(0, c0, c1); max_part(1, c0, c1); }
        if (g == 1) { max_part(2, c0, c1); max_part(3, c0, c1); }
        if (g == 2) { max_combine(); tile_ref(); }
        if (g == 3) advance(alpha, nb);
      } else {
        if (g == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) max_part(q, c0, c1);
        }
        if (g == 1) { max_combine(); tile_ref(); advance(alpha, nb); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // phase B: per M tile one V operand for the hi and the lo product
    constexpr int NB = 2 * NMT;
    i32x8 vop = vread(vslot, 0), vop_hold = {};
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int mt = i / 2;
      if (i % 2 == 0) {
        const i32x8 av = vop;
        if (mt + 1 < NMT) vop = vread(vslot, mt + 1);
        oacc[mt] = mfma_f8(av, PH[nxt], oacc[mt]);
        vop_hold = av;
      } else {
        oacc[mt] = mfma_f8(vop_hold, PL[nxt], oacc[mt]);
      }
      // the 8 exponential units: one per chunk at d = 128 (unit k's three
      // stages in chunks k, k+1 and k+2, clamped to the last), spread over the
      // 4 chunks at d = 64
      if constexpr (D == 128) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k == i) unit_fma(k, c0, c1, nb);
          if (min(k + 1, NB - 1) == i) unit_exp(k);
          if (min(k + 2, NB - 1) == i) unit_sum_pack(k, PH[cur], PL[cur]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k * NB / 8 == i) exp_unit(k, c0, c1, PH[cur], PL[cur], nb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float e = pe[0] + pe[1];
    lexact = lexact * alpha + e;
    lsteady = lsteady * alpha + e;
    pin(PH[cur]);
    pin(PL[cur]);
    pin(lexact);
    step_barrier<2 * NV_STEP>();
    rescale(alpha);
  };

  // ---- epilogue of an item: O / l (l: the sum of hi + lo, so the 2^8
  // cancels), lse = lse_scale * ref + ln(l_exact / 2^8).  finish() puts this
  // wave's O rows in its staging area (the 16-bit kernel's layout: chunk c of
  // row r at c xor ((r / rows per 256 bytes) mod chunks per row), 8-byte halves
  // swapped when r / 16 is odd); flush() stores them as whole rows after the
  // next item's prologue wait.
  constexpr int OCPR = ORB / 16;               // 16-byte chunks per O row
  constexpr int ORPB = 256 / ORB;              // O rows per 256 bytes (1 or 2)
  char* const stg = smem + 2 * kRing * BLK + w * SB;
  __bf16* o_rows = nullptr;
  float* lse_rows = nullptr;
  int o_nrows = 0;
  float lse_out = 0.0f;
  auto finish = [&]() {
    const float l = ledge + pair_reduce(lsteady, [](float x, float y) { return x + y; });
    const float le = pair_reduce(lexact, [](float x, float y) { return x + y; });
    const float inv = l > 0.0f ? a.o_scale / l : 0.0f;
    int sr = ln;
    asm volatile("" : "+v"(sr));   // addresses formed here, not hoisted
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int u = 0; u < 4; ++u) ov[u] = (__bf16)(oacc[mt][4 * g + u] * inv);
        *(bf16x4*)(stg + sr * ORB + 16 * ((4 * mt + g) ^ ((sr / ORPB) % OCPR)) + 8 * (hf ^ ((sr >> 4) & 1))) = ov;
      }
    const int wq0 = q0 + 32 * w;
    o_rows = (__bf16*)a.o + head + (size_t)wq0 * D;
    lse_rows = a.lse == nullptr ? nullptr : a.lse + (size_t)bh * N + wq0;
    o_nrows = max(0, min(32, N - wq0));
    lse_out = le > 0.0f ? a.lse_scale * st.ref + (__logf(le) - (float)kF8PreScaleLog2 * 0.69314718f)
                        : -__builtin_inff();
    count_tiles<X, FB_AUTO>(a, st, lane, qrow);
  };
  auto flush = [&]() {
    constexpr int RPI = 64 / OCPR;
    int L = lane;
    asm volatile("" : "+v"(L));
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = k * RPI + L / OCPR, cc = L % OCPR;
      u32x4 v = *(const u32x4*)(stg + r * ORB + 16 * (cc ^ ((r / ORPB) % OCPR)));
      if ((r >> 4) & 1) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);
      if (r < o_nrows) *(u32x4*)(o_rows + (size_t)r * D + 8 * cc) = v;
    }
    if (lse_rows != nullptr && hf == 0 && ln < o_nrows) lse_rows[ln] = lse_out;
  };

  int it = item_of(0, gid, nwg);
  set_item(it);
  bool pref = false;
  for (int round = 0;; ++round) {
    const int it_next = item_of(round + 1, gid, nwg);
    set_next(it_next);
    if (!pref) {
      load_q(head, qrow, qvalid);
#pragma unroll
      for (int j = 0; j < kKAhead; ++j) load_k(j, Int<0>());
#pragma unroll
      for (int j = 0; j < kVAhead; ++j) load_v(j, Int<0>());
    }
    step_barrier<0>();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), as the compiler sees it (Q loaded)
    if (round > 0) flush();

    row_state_init(st, X == 1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) oacc[mt] = f32x16{};
    ledge = 0.0f;
    lsteady = 0.0f;
    lexact = 0.0f;
    S[0][0] = S[0][1] = S[1][0] = S[1][1] = f32x16{};
    PH[0] = PH[1] = PL[0] = PL[1] = i32x8{};
    if (jend_w > 0) qk(0, S[0][0], S[0][1]);
    // step 0 refills K_0's slot (the O stores may stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    int j = 0;
    edge_step(j++);
    for (; j + 8 <= jend_w; j += 4) {
      steady_step(Int<0>(), j, Int<0>());
      steady_step(Int<1>(), j + 1, Int<0>());
      steady_step(Int<2>(), j + 2, Int<0>());
      steady_step(Int<3>(), j + 3, Int<0>());
    }
    if (j + 4 < jend_w) {
      steady_step(Int<0>(), j, Int<1>());
      steady_step(Int<1>(), j + 1, Int<1>());
      steady_step(Int<2>(), j + 2, Int<1>());
      steady_step(Int<3>(), j + 3, Int<1>());
      j += 4;
    }
    if (j + 2 < jend_w) {
      steady_step(Int<0>(), j, Int<1>());
      steady_step(Int<1>(), j + 1, Int<1>());
      j += 2;
    }
    for (; j <= jend; ++j) edge_step(j);
    // zero loads past the item's end land before the next item reuses the slots
    if (!pref_next) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    finish();
    if (it_next >= nitems) {
      flush();
      break;
    }
    pref = pref_next;
    it = it_next;
    set_item(it);
  }
}

}  // namespace tos
