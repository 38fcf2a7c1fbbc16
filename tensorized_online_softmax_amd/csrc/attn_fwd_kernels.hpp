// attn_fwd_kernels.hpp -- fused attention forward kernels for gfx950 (MI355X):
// attn_fwd_h16 (bf16 and fp16 inputs: persistent 8-wave workgroups of 256
// query rows, 64-key blocks in LDS rings; described at its definition) and
// attn_fwd_f32 (fp32 inputs: 4-wave workgroups of 128 query rows, one 64-key
// block at a time in LDS).  attn_fwd_fp8.hpp holds the fp8 kernel.
//
// In both, each wave owns 32 query rows, and per key block each wave runs the
// fused-attention iteration of FlashAttention-T
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

#include "pieces.hpp"
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

// 16-bit element types of the second kernel family: bf16 and fp16 share the
// 32x32x16 MFMA shape, the transposing 16-bit LDS read and every layout; only
// the MFMA, the dot product with (1, 1) and the conversions differ.
template <typename E> struct Elem16;
template <> struct Elem16<__bf16> {
  // P~ <= 1 is packed as is: bf16 keeps float32's exponent range
  static constexpr int kPreLog2 = 0;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <> struct Elem16<_Float16> {
  // fp16 has normals only down to 2^-14: P~ is packed as P~ * 2^15 (at most
  // 2^15 < 65504, since the reference is at least the row's maximum), so that a
  // row 29 log2-units below its tile's surrogate still packs normal numbers.
  // The factor cancels in O / l and is taken out of lse.
  static constexpr int kPreLog2 = 15;
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;            // batch * heads
  int N;             // sequence length
  int nqb;           // query blocks per head (set by the launcher for its block size)
  float c;           // scale * log2(e) (fp8: times the q and k descales)
  float lse_scale;   // scale (fp8: times the q and k descales)
  float o_scale;     // multiplies O at the end (fp8: the v descale)
  float tau;         // fallback threshold, log2 units
  int* fallback_tiles;   // per-row tile counter, or nullptr
  int count_x;       // > 0: count the X-row tiles of this size as per-row (FORCE)
  // 16-bit kernels: items cut into pieces of at most split_c key blocks
  // (pieces.hpp; 0 = whole items), nunits work units in all, and the
  // workspace of the pieces' partial results (piece_bytes(d) per unit)
  int split_c;
  int nunits;
  float* ws;
  unsigned long long* trace;   // traced instances: per-wave phase cycles (kTraceSlots each)
};

// Phase accounting of the traced instances (TRACE = true): per wave, in
// s_memtime cycles, slots of trace[(workgroup * 8 + wave) * kTraceSlots + i]:
constexpr int kTraceSlots = 16;
enum TraceSlot {
  kTrWave = 0,       // from the wave's first stamp to its last
  kTrSteadyN = 1,    // steady steps
  kTrSteady = 2,     // their cycles, barrier to barrier
  kTrPhaseA = 3,     //   phase A (S_{j+1} = K Q^T with the first units)
  kTrPhaseB = 4,     //   phase B (P~V with the remaining units), up to the barrier
  kTrSteadyWait = 5, //   the barrier
  kTrEdgeN = 6,      // edge steps (first, last and idle steps of a wave)
  kTrEdge = 7,       // their cycles
  kTrEdgeSoftmax = 8,  //   the softmax section, before the step's matrix instructions
  kTrEdgeWait = 9,   //   the barrier
  kTrRealtime = 10,  // kTrWave's span in s_memrealtime ticks (a fixed 100 MHz clock)
  kTrRtFirst = 11,   // s_memrealtime at the wave's first and last stamps (one clock
  kTrRtLast = 12     // for the whole chip: the launch's span and each wave's place in it)
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

// Items of the persistent kernels: item i is query block qb of head bh, with
// bh = i mod BH and the blocks numbered heaviest first when causal (the query
// blocks with the most keys).
__device__ __forceinline__ void item_coords(const FwdArgs& a, bool causal, int i, int& bh, int& qb) {
  bh = i % a.BH;
  qb = causal ? (a.nqb - 1 - i / a.BH) : i / a.BH;
}

// The item that workgroup g of G runs in round r.  Even rounds deal items in
// order, odd rounds deal them backwards in groups of 8 workgroups, so that a
// workgroup that got one of the heavier items of a round gets one of the
// lighter ones of the next (causal work evens out), while workgroup g still
// gets items of the heads h = g mod 8 (mod 8): with G and BH multiples of 8,
// the items of a head stay on the XCD that workgroup g runs on (workgroups are
// dealt to the 8 XCDs round-robin), where its K and V stay in L2.
// (A G that is not a multiple of 8 deals every round in order.)
__device__ __forceinline__ int item_of(int r, int g, int G) {
  const int gg = ((r & 1) && (G & 7) == 0) ? (G - 8 - (g & ~7)) + (g & 7) : g;
  return r * G + gg;
}

// Tile counter: once per tile that ran with per-row maxima.
template <int X, bool FB_AUTO>
__device__ __forceinline__ void count_tiles(const FwdArgs& a, const RowState& st, int lane,
                                            int qrow) {
  if (a.fallback_tiles == nullptr || lane >= 32 || qrow >= a.N) return;
  if constexpr (FB_AUTO) {
    if (st.per_row && (qrow % X) == 0) atomicAdd(a.fallback_tiles, 1);
  } else {
    if (a.count_x > 0 && (qrow % a.count_x) == 0) atomicAdd(a.fallback_tiles, 1);
  }
}

// ---------------------------------------------------------------------------
// 16-bit inputs (bf16, fp16): v_mfma_f32_32x32x16_{bf16,f16} for both
// products, software-pipelined.  (Below, "bf16" stands for either.)
//
// A workgroup has 8 waves = 256 query rows (waves w and w+4 share a SIMD) and
// one LDS ring of key blocks.  Each wave runs its own three-stage pipeline: in
// the step for key block j it issues, in one instruction stream,
//   matrix unit : O^T += V_{j-1}^T P~_{j-1}^T   and   S_{j+1} = K_{j+1} Q^T
//   vector units: the softmax of S_j -> P~_j (tile max, exp2, pack, row sums)
// with the MFMAs spread between the vector instructions, so that the tensor
// and vector work of FlashAttention-T (section A2, tensor-vector scheduling)
// overlap inside the wave, and the second wave on the SIMD fills what one wave
// leaves idle.  The rescale of O by alpha_j (rare: the surrogate maximum
// seldom moves) comes after the P~_{j-1} product and before the P~_j one.
//
// Key blocks stream into two LDS rings of 4 slots (K and V) through buffer
// loads that write LDS directly (no registers; rows past N read as 0).  Step j
// issues K_{j+4} and V_{j+2} into the slots that K_j and V_{j-2} held (read in
// step j-1); blocks past an item's last one are the next item's first ones
// (see below) or zeros, so every step issues the same loads.  Every step ends
// with a plain barrier after waiting until only the loads of the last two
// steps are in flight.
//
// The launch is persistent: one workgroup per compute unit, each running a
// static list of items (256-row query blocks of a head, heaviest first, see
// item_of).  The rings run on across items, the next item's Q is loaded in
// the last step of the current one, and O leaves through LDS as whole rows
// after the next item's prologue wait.
// A direct-to-LDS load writes 1 KiB per wave instruction, contiguous, so rows
// are not padded: 16-byte chunks are XOR-swizzled within each row instead,
// which keeps the K operand reads (16 rows, one chunk each) and the
// transposing V reads (4 rows x 2 chunks per 16 lanes) free of bank conflicts.
//
// Steady steps run four to a loop iteration (the ring period), so that ring
// slots are constants folded into the LDS instructions, and S and P~ alternate
// between two register sets instead of being copied.
// ---------------------------------------------------------------------------
constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPBr = 32 * kPWaves;   // 256 query rows per workgroup
constexpr int kRing = 4;             // LDS ring slots for K and for V
constexpr int kKAhead = 4;           // step j loads K_{j+4}
constexpr int kVAhead = 2;           // step j loads V_{j+2}

// Raw buffer descriptor (stride 0) over [base, base + bytes): loads at offsets
// at or past `bytes` return zeros.  The fourth word is the gfx9 data format
// for untyped dword loads.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((unsigned)b);
  d[1] = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// Descriptor of key block j (blk bytes each) of a head: the buffer moved to
// the block's start, or, for j >= jlim, an empty one (every load reads zeros).
__device__ __forceinline__ u32x4 block_desc(u32x4 d, int j, int jlim, unsigned blk) {
  const unsigned off = (unsigned)j * blk;
  const unsigned long long b = ((unsigned long long)d[1] << 32 | d[0]) + (j < jlim ? off : 0u);
  u32x4 r;
  r[0] = (unsigned)b;
  r[1] = (unsigned)(b >> 32) & 0xffffu;
  r[2] = j < jlim ? d[2] - off : 0u;
  r[3] = d[3];
  return r;
}

// c ? x : y for wave-uniform descriptors, as scalar selects (the compiler
// would otherwise branch around the computation of the one not taken)
__device__ __forceinline__ u32x4 select_desc(bool c, u32x4 x, u32x4 y) {
  // (the operands are uniform; readfirstlane says so where the compiler
  // cannot prove it, and is free where it can)
  const unsigned cc = __builtin_amdgcn_readfirstlane((unsigned)c);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned v;
    asm("s_cmp_lg_u32 %1, 0\n\ts_cselect_b32 %0, %2, %3"
        : "=s"(v)
        : "s"(cc), "s"(__builtin_amdgcn_readfirstlane(x[i])), "s"(__builtin_amdgcn_readfirstlane(y[i]))
        : "scc");
    r[i] = v;
  }
  return r;
}

// LDS position (16-byte chunk index within the row) of chunk c of row r
template <int D> __device__ __forceinline__ int kswz(int r, int c) {
  return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}
template <int D> __device__ __forceinline__ int vswz(int r, int c) {
  return D == 128 ? (c ^ (4 * (r & 3))) : (c ^ (4 * ((r >> 1) & 1)));
}

// NW direct-to-LDS loads of 1 KiB each: instruction k writes LDS bytes
// [lds + 1024k, +1024) (16 bytes per lane, in lane order) from the byte offsets
// goff[k] of the buffer `desc`.  `lds` is a wave-uniform LDS byte address.
//
// Issued from inline assembly on purpose: the compiler cannot tell which LDS
// bytes a direct-to-LDS load writes, so after the builtin form it makes the
// next LDS read wait for every load in flight, which would serialise each
// step's prefetch with that step's own reads.  These loads write ring slots
// that no wave reads before the step_barrier that waits for them (its vmcnt
// count covers these loads), so no such wait is needed.  M0 holds the LDS
// destination; it is saved and restored around the loads, and one wait state
// separates its write from the load that reads it.
template <int NW>
__device__ __forceinline__ void dma_block(u32x4 desc, unsigned lds, const unsigned* goff) {
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds + 1024u * k), "v"(goff[k]), "s"(desc));
  }
}

// end of a step: wait until at most NV vector-memory loads of this wave are in
// flight and its LDS reads are done, then the workgroup barrier.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
template <int NV> __device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NV) : "memory");
}

// keeps x in registers here: the computation of x cannot sink past this point.
// (Device pass only: kernel lambdas are also parsed for the host, where a
// vector-register operand of this width does not exist.)
template <typename T> __device__ __forceinline__ void pin(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#else
  (void)x;
#endif
}

template <int I> struct Int { static constexpr int value = I; };

// Split plan of the element-wise softmax steps between the matrix unit and the
// vector unit (FlashAttention-T, section A2: repurposed matrix instructions for
// scaling / FMA (Fig 5(a)) and the row sum (Fig 5(b)); "tensor-vector split":
// horizontal within a tile (Fig 6(a)) or vertical across a wave's tiles
// (Fig 6(b))).  One int, fixed at compile time:
//   bits 0-2   rs: of the 4 sixteen-key steps of a key block, those below rs
//              take their row sum on the matrix unit (ones x P~^T)
//   bits 3-7   z:  Z = c*S - c*ref on the matrix unit (f32 products against
//              c*I, the offset -c*ref added by one more product): register
//              slices s < z of both 32x32 S tiles (horizontal), or tiles t < z
//              (vertical)
//   bits 8-12  o:  the O rescale on the matrix unit (f32 products against
//              alpha*I): slices s < o of every 32x32 O tile (horizontal), or
//              tiles mt < o (vertical)
//   bit 13     vertical
// 0 is the all-vector plan.
constexpr int split_plan(int rs, int z, int o, bool vertical) {
  return rs | (z << 3) | (o << 8) | ((int)vertical << 13);
}
constexpr int plan_rs(int P) { return P & 7; }
constexpr int plan_z(int P) { return (P >> 3) & 31; }
constexpr int plan_o(int P) { return (P >> 8) & 31; }
constexpr bool plan_vert(int P) { return (P >> 13) & 1; }
// register slice s of S tile t / of O tile mt on the matrix unit?
constexpr bool z_on_mfma(int P, int t, int s) { return plan_vert(P) ? t < plan_z(P) : s < plan_z(P); }
constexpr bool o_on_mfma(int P, int mt, int s) { return plan_vert(P) ? mt < plan_o(P) : s < plan_o(P); }
constexpr bool rs_on_mfma(int P, int step) { return step < plan_rs(P); }
constexpr int kPlanValu = 0;
constexpr int kPlanRowsumMfma = split_plan(4, 0, 0, false);
constexpr int kPlanScaleMfma = split_plan(0, 0, 16, false);


// SEQ: the sequential-schedule ablation -- every step is the generic step
// (softmax, then QK^T, then P~V), with no interleaving inside a wave.
// PLAN: the split plan (split_plan above).  A plan that puts O rescale slices
// on the matrix unit needs one alpha per wave (X = 32, no per-row fallback).
// TRACE: phase stamps (s_memtime, each followed by a wait for it, at points where
// no LDS read is pending or about to be waited for) accumulated per wave into
// a.trace, for the vector-interval accounting; an instrumented copy, slower.
template <typename E, int D, bool CAUSAL, int X, int PLAN, bool FB_AUTO, bool SEQ, bool TRACE = false>
__global__ __launch_bounds__(kPThreads, 1) void attn_fwd_h16(FwdArgs a) {
  constexpr int RS = plan_rs(PLAN);                   // row-sum steps on the matrix unit
  constexpr bool ROWSUM_ANY = RS > 0, ROWSUM_ALL = RS == 4;
  constexpr bool Z_ANY = plan_z(PLAN) > 0, O_ANY = plan_o(PLAN) > 0;
  static_assert(!O_ANY || (X == 32 && !FB_AUTO), "matrix-unit O rescale needs one alpha per wave");
  static_assert(plan_vert(PLAN) || plan_z(PLAN) % 2 == 0, "Z slices come in pairs (one unit each)");
  typedef typename Elem16<E>::v8 ev8;
  typedef typename Elem16<E>::v4 ev4;
  typedef typename Elem16<E>::v2 ev2;
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int RB = 2 * D;                   // bytes per K or V row
  constexpr int BLK = kBc * RB;               // bytes per key block of K or V
  constexpr int CHW = BLK / 1024 / kPWaves;   // 1 KiB load instructions per wave per tensor
  constexpr int NKK = D / 16;                 // k-steps of S^T = K Q^T
  constexpr int NMT = D / 32;                 // 32-row M tiles of O^T
  constexpr int NV_STEP = 2 * CHW;            // loads a wave issues per step
  // V ring first: its slot offsets plus the in-block offsets fit the 16-bit
  // immediate of the LDS reads; the K ring's base is folded into koff
  // Past the rings, 4 x 32 rows of O staging: each wave transposes its O tile
  // through LDS (32 rows, waves 0-3 in V slots 2 and 3, free then, waves 4-7
  // here) so that the stores write whole rows.
  constexpr int SB = 32 * RB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kRing * BLK + 4 * SB];
  char* vring = smem;

  // the wave index is the same in every lane: say so, so that everything
  // derived from it (block ranges, LDS slots, descriptors) stays scalar
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Persistent workgroups: workgroup g of G runs units item_of(0, g),
  // item_of(1, g), ... until they run out.  A unit is an item (a query block of
  // a head) or, with a.split_c > 0, a piece of one: a range of its key blocks
  // (pieces.hpp), whose partial O and lse go to the workspace.
  const int N = a.N;
  const int nblk = (N + kBc - 1) / kBc;
  const int nunits = a.nunits;
  const int nwg = gridDim.x, gid = blockIdx.x;

  // the current unit (wave-uniform, but qrow, qvalid and klim); key blocks are
  // counted from the unit's first one, jb0
  int bh = 0, q0 = 0, qrow = 0, jend = 0, jend_w = 0, klim = 0, jb0 = 0, unit = 0;
  bool qvalid = false, part = false;
  size_t head = 0;
  u32x4 kdesc = {}, vdesc = {};
  // K (V) of head bh from key block jb on: rows past N read as zeros
  auto kv_desc = [&](const void* base, size_t head_, int jb) {
    return buffer_desc((const E*)base + head_ + (size_t)jb * kBc * D, (unsigned)(N - jb * kBc) * RB);
  };
  auto set_item = [&](int it) {
    const Piece pc = piece_of(it, a.BH, a.nqb, N, CAUSAL, a.split_c);
    bh = pc.bh;
    q0 = pc.qb * kPBr;
    jb0 = pc.jb;
    unit = it;
    part = pc.np > 1;
    qrow = q0 + 32 * w + ln;
    qvalid = qrow < N;
    head = (size_t)bh * N * D;
    kdesc = kv_desc(a.k, head, jb0);
    vdesc = kv_desc(a.v, head, jb0);
    jend = pc.je - pc.jb;
    // first query of the wave (X = 64: of its pair of waves, which must step
    // through the same key blocks to exchange their tile maxima), and the
    // wave's key blocks within the unit's
    const int wq0 = X == 64 ? q0 + 64 * (w / 2) : q0 + 32 * w;
    const int wrows = X == 64 ? 64 : 32;
    const int wend = (wq0 >= N) ? 0 : (CAUSAL ? min(wq0 + wrows - 1, N - 1) / kBc + 1 : nblk);
    jend_w = max(0, min(wend, pc.je) - pc.jb);
    klim = qvalid ? (CAUSAL ? qrow + 1 : N) : 0;       // keys this lane may see
  };
  // The next unit's first K and V blocks are loaded by this unit's last steps
  // (the ring continues across units) when this unit's block count is a
  // multiple of the ring size, so that those blocks land in the slots the
  // next unit expects them in.
  // Its Q fragments are loaded in this unit's last step, after the last use
  // of this unit's.
  bool pref_next = false;
  int jend_n = 0, qrow_n = 0;
  bool qvalid_n = false;
  size_t head_n = 0;
  u32x4 kdesc_n = {}, vdesc_n = {};
  auto set_next = [&](int it) {
    pref_next = it < nunits && jend % kRing == 0;
    if (pref_next) {
      const Piece pc = piece_of(it, a.BH, a.nqb, N, CAUSAL, a.split_c);
      head_n = (size_t)pc.bh * N * D;
      kdesc_n = kv_desc(a.k, head_n, pc.jb);
      vdesc_n = kv_desc(a.v, head_n, pc.jb);
      jend_n = pc.je - pc.jb;
      qrow_n = pc.qb * kPBr + 32 * w + ln;
      qvalid_n = qrow_n < N;
    }
  };

  // Q^T operand: lane (query ln, half hf) holds Q[qrow][16 kk + 8 hf + 0..7]
  ev8 qf[NKK];
  auto load_q = [&](size_t head_, int qrow_, bool qvalid_) {
    const E* Q = (const E*)a.q + head_;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qvalid_)
        qf[kk] = *(const ev8*)(Q + (size_t)qrow_ * D + 16 * kk + 8 * hf);
      else
        qf[kk] = ev8{};
    }
  };

  // direct-to-LDS loads: instruction k of this wave fills LDS bytes
  // [(w*CHW + k)*1024, +1024) of the slot, lane L the 16 bytes at +16L, i.e.
  // row r, chunk position p; it fetches chunk c = p xor swizzle(r) of row r
  unsigned kgoff[CHW], vgoff[CHW];
#pragma unroll
  for (int k = 0; k < CHW; ++k) {
    const int L = (w * CHW + k) * 1024 + 16 * lane, r = L / RB, p = (L % RB) / 16;
    kgoff[k] = (unsigned)(r * RB + 16 * kswz<D>(r, p));
    vgoff[k] = (unsigned)(r * RB + 16 * vswz<D>(r, p));
  }
  // wave-uniform LDS byte addresses of this wave's share of ring slot 0
  const unsigned lds0 = (unsigned)(unsigned long long)(__attribute__((address_space(3))) char*)smem;
  const unsigned vdst = lds0 + (unsigned)w * CHW * 1024, kdst = vdst + kRing * BLK;
  // block j of the item's K (V), zeros past its end; with XING (a step that
  // may cross the item's end) the blocks past the end are the next item's
  // first ones when those are prefetched
  auto ring_desc = [&](const u32x4& cur, const u32x4& nxt, int j) -> u32x4 {
    return select_desc(pref_next & (j >= jend), block_desc(nxt, j - jend, jend_n, BLK),
                       block_desc(cur, j, jend, BLK));
  };
  auto load_k = [&](int j, auto XING) {
    if constexpr (decltype(XING)::value)
      dma_block<CHW>(ring_desc(kdesc, kdesc_n, j), kdst + (j % kRing) * BLK, kgoff);
    else
      dma_block<CHW>(block_desc(kdesc, j, jend, BLK), kdst + (j % kRing) * BLK, kgoff);
  };
  auto load_v = [&](int j, auto XING) {
    if constexpr (decltype(XING)::value)
      dma_block<CHW>(ring_desc(vdesc, vdesc_n, j), vdst + (j % kRing) * BLK, vgoff);
    else
      dma_block<CHW>(block_desc(vdesc, j, jend, BLK), vdst + (j % kRing) * BLK, vgoff);
  };

  // K operand reads: lane (key ln of tile t, half hf) reads chunk 2kk + hf of
  // row 32t + ln; the swizzle depends on the row only through ln
  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = kRing * BLK + ln * RB + 16 * kswz<D>(ln, 2 * kk + hf);
  // V transposing reads: lane (16-lane group G, index i) reads 8 bytes of row
  // 16s + 4(G/2) + i/4 (+8 for slots 4..7) at element 32mt + 16(G%2) + 4(i%4),
  // i.e. chunk 4mt + 2(G%2) + (i%4)/2, byte 8((i%4)%2) within it
  const int G = lane >> 4, gi = lane & 15;
  const int vr0 = 4 * (G >> 1) + (gi >> 2);
  int voff[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
    voff[mt] = vr0 * RB + 16 * vswz<D>(vr0, 4 * mt + 2 * (G & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);

  RowState st;
  const float c = a.c, tau = a.tau;
  f32x16 oacc[NMT];
  float lsum;       // row sum of the rounded P~ over the steps the vector unit
                    // takes (this lane's keys only)
  f32x16 lacc;      // the same over the matrix unit's steps (every register
                    // holds the full sum)
  float lexact;     // row sum of the unrounded P~ (this lane's keys only)
  // Pipeline registers: entering step j, S_j in S[0] and P~_{j-1} in P[1]
  // (the steady steps alternate the two sets)
  f32x16 S[2][2];
  ev8 P[2][4];
  ev8 ones;
#pragma unroll
  for (int t = 0; t < 8; ++t) ones[t] = (E)1.0f;
  const ev2 ones2 = {(E)1.0f, (E)1.0f};

  // ---- operands and single matrix instructions
  // QK instruction g (0 <= g < NQK) of S^T = K Q^T: key tile t = g % 2,
  // k-step kk = g / 2; its K operand comes from the K block at kt
  constexpr int NQK = 2 * NKK, NPV = 4 * NMT;
  auto kread = [&](const char* kt, int g) -> ev8 {
    return *(const ev8*)(kt + koff[g / 2] + (g % 2) * 32 * RB);
  };
  auto qk_mfma = [&](int g, ev8 av, f32x16& t0, f32x16& t1) {
    f32x16& acc = (g % 2) ? t1 : t0;
    acc = Elem16<E>::mfma(av, qf[g / 2], g < 2 ? f32x16{} : acc);
  };
  // PV instruction i (0 <= i < NPV) of O^T += V^T P~^T: 16-key step s = i / NMT,
  // M tile mt = i % NMT.  Step s, slot t of lane half h is key
  // 16s + 8(t/4) + 4h + t%4 (the accumulator order of S^T), which the
  // transposing reads fetch.
  auto vread = [&](const char* vt, int i) -> ev8 {
    const char* p = vt + voff[i % NMT] + 16 * (i / NMT) * RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 8 * RB));
    return __builtin_bit_cast(ev8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv_mfma = [&](int i, ev8 av, const ev8* pk) {
    oacc[i % NMT] = Elem16<E>::mfma(av, pk[i / NMT], oacc[i % NMT]);
    if constexpr (ROWSUM_ANY)   // step 7 on the matrix unit: ones x P~^T
      if (i % NMT == NMT - 1 && rs_on_mfma(PLAN, i / NMT))
        lacc = Elem16<E>::mfma(ones, pk[i / NMT], lacc);
  };
  auto qk = [&](int slot, f32x16& t0, f32x16& t1) {
    const char* kt = smem + slot * BLK;
#pragma unroll
    for (int g = 0; g < NQK; ++g) qk_mfma(g, kread(kt, g), t0, t1);
  };
  auto pv = [&](int slot, const ev8* pk) {
    const char* vt = vring + slot * BLK;
#pragma unroll
    for (int i = 0; i < NPV; ++i) pv_mfma(i, vread(vt, i), pk);
  };

  // ---- phase stamps (TRACE)
  unsigned long long tr[kTraceSlots] = {};
  unsigned long long t_first = 0, t_last = 0, rt_first = 0;
  auto realtime = [&]() -> unsigned long long {
    unsigned long long t;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
    return t;
  };
  // (branch-free: the wave's first stamps are taken once, before its first unit)
  auto stamp = [&]() -> unsigned long long {
    if constexpr (TRACE) {
      unsigned long long t;
      asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
      t_last = t;
      return t;
    } else {
      return 0;
    }
  };

  // ---- the softmax of one key block, in pieces (Algorithm 1)
  // Key of register r of tile t in block j: j*Bc + 32t + 8(r/4) + 4hf + r%4.
  // Only a wave's last block can hold keys past the diagonal or past N.
  auto mask_block = [&](int j, f32x16& s0, f32x16& s1) {
    const int kb = (jb0 + j) * kBc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + 8 * (r / 4) + 4 * hf + (r % 4);
      if (key >= klim) s0[r] = -__builtin_inff();
      if (key + 32 >= klim) s1[r] = -__builtin_inff();
    }
  };
  // step 1, in four chains of 8 logits: part q covers registers 8q'..8q'+7
  // of tile q/2 (q' = q % 2)
  float bm4[4];
  auto max_part = [&](int q, const f32x16& s0, const f32x16& s1) {
    const f32x16& sv = (q / 2) ? s1 : s0;
    const int r0 = 8 * (q % 2);
    // one v_max3 per two logits (the compiler would build a tree of v_max
    // and v_max3 instead: 5 instructions per 8 logits rather than 4)
    float m = fmax_raw(sv[r0], sv[r0 + 1]);
#pragma unroll
    for (int r = r0 + 2; r < r0 + 8; r += 2) m = fmax3_raw(m, sv[r], sv[r + 1]);
    bm4[q] = m;
  };
  // steps 2-3: running row maxima and the lane-pair combine; rows past N stay
  // out of the tile maximum
  auto max_combine = [&]() {
    float bm = fmax_raw(fmax3_raw(bm4[0], bm4[1], bm4[2]), bm4[3]);
    bm = qvalid ? bm : -__builtin_inff();
    row_max_update(st, bm);
  };
  // the tile maximum (the surrogate) and the new reference: alpha, and
  // -c * ref for the exponentials
  float ref_new = 0.0f;
  // X = 64: the tile is waves 2p and 2p+1.  Each publishes the maximum (and,
  // with AUTO, the minimum) of its 32 rows' running maxima in LDS under a
  // per-block sequence number and takes its partner's; the partner cannot be a
  // block ahead (the step barrier), so the slot holds this block's value or
  // the last one.  The wait is bounded: past it the wave keeps its own half
  // (any reference at least the rows' maxima gives the same result).  The
  // slots are the last 128 bytes of wave 7's O staging area, which that wave's
  // row 31 bypasses.
  float* const xslot = (float*)(smem + 2 * kRing * BLK + 4 * (32 * RB) - 128);
  int xseq = 0;
  auto tile_ref = [&]() {
    if constexpr (X == 64) {
      const float ninf = -__builtin_inff();
      const float own = tile_reduce<32>(st.m_run, MaxOp());
      const float own_mn = FB_AUTO ? tile_reduce<32>(st.m_run == ninf ? __builtin_inff() : st.m_run, MinOp())
                                   : 0.0f;
      ++xseq;
      float* mine = xslot + 4 * w;
      if (lane == 0) {
        mine[0] = own;
        mine[1] = own_mn;
        __hip_atomic_store((int*)(mine + 2), xseq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      const float* other = xslot + 4 * (w ^ 1);
      float pmx = own, pmn = own_mn;
      int tries = 0;
      while (__hip_atomic_load((const int*)(other + 2), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != xseq &&
             ++tries < (1 << 16))
        __builtin_amdgcn_s_sleep(1);
      if (tries < (1 << 16)) {
        pmx = other[0];
        pmn = other[1];
      }
      ref_new = ref_from_tile<FB_AUTO>(st, fmax_raw(own, pmx), fmin_raw(own_mn, pmn), c, tau);
    } else {
      ref_new = block_ref<X, FB_AUTO>(st, c, tau);
    }
  };
  auto advance = [&](float& alpha, float& nb) {
    alpha = ref_advance(st, ref_new, c);
    nb = neg_c_ref(st, c) + (float)Elem16<E>::kPreLog2;
  };
  // the same in a steady step of a wave-wide tile without fallback: every row of
  // the wave has seen key block 0 by then, so the old and the new reference are
  // finite and the guards of ref_advance / neg_c_ref are not needed
  auto advance_steady = [&](float& alpha, float& nb) {
    if constexpr (X == 32 && !FB_AUTO) {
      alpha = __builtin_amdgcn_exp2f(c * (st.ref - ref_new));
      st.ref = ref_new;
      nb = __builtin_fmaf(-c, ref_new, (float)Elem16<E>::kPreLog2);
    } else {
      advance(alpha, nb);
    }
  };
  // steps 4-7 for registers r, r+1 of tile t (unit k: t = k / 8,
  // r = 2 (k % 8)): P~ = exp2(c*S - c*ref), packed to 16 bits as the B operand
  // of the P~V product, and both row sums.  The unrounded sum gives lse; the
  // sum of the rounded P~ that the product consumes normalises O, so O / l
  // stays a weighted average of V rows (16-bit rounding of P~ then cancels to
  // first order instead of adding to the error of O).
  // A unit runs in three stages, so that a steady step can issue them in
  // different chunks and keep each stage's inputs ready when it issues:
  // (1) the FMA Z = c*S - c*ref, (2) exp2, (3) both sums and the packing.
  float pe[2], ps[2];
  float uz[16][2], up[16][2];   // per unit: Z, then P~ (registers, unrolled)
  auto sums_reset = [&]() { pe[0] = pe[1] = ps[0] = ps[1] = 0.0f; };
  auto unit_fma = [&](int k, const f32x16& s0, const f32x16& s1, float nb) {
    const int t = k / 8, r = 2 * (k % 8);
    const f32x16& sv = t ? s1 : s0;
    uz[k][0] = __builtin_fmaf(sv[r], c, nb);
    uz[k][1] = __builtin_fmaf(sv[r + 1], c, nb);
  };
  // Z on the matrix unit (the plan's slices, steady steps only: the S of a
  // steady step holds no masked -inf logit, which a zero of the selection
  // operand would turn into NaN).  Per 32x32 tile, one chain of f32 products
  // into zacc[t]: first the offset (lane half 0 passes 1 against -c*ref, half
  // 1 passes 0, so every row of column n gets -c*ref of query n), then slice s
  // as the B operand against c times the columns of I that pick its rows
  // (rows 8(s/4) + 4h + s%4 of lane half h), the selection precomputed once.
  f32x16 zacc[2];
  float zsel[16];
#pragma unroll
  for (int sl = 0; sl < 16; ++sl)
    zsel[sl] = (Z_ANY && (z_on_mfma(PLAN, 0, sl) || z_on_mfma(PLAN, 1, sl)) &&
                ln == 8 * (sl / 4) + 4 * hf + sl % 4) ? c : 0.0f;
  const float zoff_sel = hf == 0 ? 1.0f : 0.0f;
  auto z_chain = [&](const f32x16& s0, const f32x16& s1, float nb) {
    if constexpr (Z_ANY) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bool any = false;
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) any = any || z_on_mfma(PLAN, t, sl);
        if (!any) continue;
        const f32x16& sv = t ? s1 : s0;
        f32x16 z = __builtin_amdgcn_mfma_f32_32x32x2f32(zoff_sel, nb, f32x16{}, 0, 0, 0);
#pragma unroll
        for (int sl = 0; sl < 16; ++sl)
          if (z_on_mfma(PLAN, t, sl)) z = __builtin_amdgcn_mfma_f32_32x32x2f32(zsel[sl], sv[sl], z, 0, 0, 0);
        zacc[t] = z;
      }
    }
  };
  // stage 1 in a steady step: the plan's slices come from the chain
  auto unit_fma_steady = [&](int k, const f32x16& s0, const f32x16& s1, float nb) {
    const int t = k / 8, r = 2 * (k % 8);
    if (z_on_mfma(PLAN, t, r)) {
      uz[k][0] = zacc[t][r];
      uz[k][1] = zacc[t][r + 1];
    } else {
      unit_fma(k, s0, s1, nb);
    }
  };
  auto unit_exp = [&](int k) {
    up[k][0] = __builtin_amdgcn_exp2f(uz[k][0]);
    up[k][1] = __builtin_amdgcn_exp2f(uz[k][1]);
  };
  // The rounded row sum (the normaliser of O) is taken on the vector unit only
  // in a wave's edge steps (its first and last key blocks, and the idle steps of
  // a causal item); a steady step adds its unrounded sum instead.  A row whose
  // keys are few (the early rows of a causal head) has all of them in edge
  // blocks, where O / l must stay an exact weighted average of V rows; a row
  // with steady blocks has more than 128 keys, over which the 16-bit rounding
  // of P~ averages out.  This drops the dot products (which wait for the
  // matrix unit to go idle) from the steady steps.  bf16 only: its P~ keeps
  // fp32's exponent range, while fp16 P~ flushes rows far below their tile's
  // surrogate, and there an unrounded sum next to a flushed numerator would
  // shrink O towards 0 instead of leaving the surviving terms' average.
  constexpr bool STEADY_EXACT = PLAN == kPlanValu && Elem16<E>::kPreLog2 == 0;
  // With the whole row sum on the matrix unit (ones x P~^T for every block,
  // the normaliser of O), a steady step takes no vector sum at all: lse then
  // uses the rounded sum of the steady blocks, plus, from the edge steps, the
  // unrounded sums of their blocks (kept as a correction: unrounded minus
  // rounded).  A row with steady blocks has more than 128 keys, and its lse
  // is then at least ln 128, where the rounding of P~ (2^-9 relative at most)
  // stays inside the relative bound of lse.
  constexpr bool LEAN = PLAN == kPlanRowsumMfma;
  auto unit_sum_pack = [&](int k, ev8* pk, bool steady) {
    const int t = k / 8, r = 2 * (k % 8);
    const float p0 = up[k][0], p1 = up[k][1];
    if (!(LEAN && steady)) {
      pe[t] += p0;
      pe[t] += p1;
    }
    ev2 w;
    w[0] = (E)p0;
    w[1] = (E)p1;
    pk[2 * t + r / 8][r % 8] = w[0];
    pk[2 * t + r / 8][r % 8 + 1] = w[1];
    if ((LEAN && !steady) || (!(steady && STEADY_EXACT) && !rs_on_mfma(PLAN, 2 * t + r / 8)))
      ps[t] = Elem16<E>::dot2(w, ones2, ps[t]);
  };
  auto exp_unit = [&](int k, const f32x16& s0, const f32x16& s1, ev8* pk, float nb) {
    unit_fma(k, s0, s1, nb);
    unit_exp(k);
    unit_sum_pack(k, pk, false);
  };
  // the block's sums into the running ones (which absorb alpha here; O and the
  // MFMA row sum get alpha at the end of the step)
  auto sums_commit = [&](float alpha, bool steady) {
    if constexpr (LEAN) {   // lexact holds the edge blocks' unrounded-minus-rounded sums
      lexact = steady ? lexact * alpha : lexact * alpha + ((pe[0] + pe[1]) - (ps[0] + ps[1]));
      return;
    }
    const float e = pe[0] + pe[1];
    lexact = lexact * alpha + e;
    if constexpr (!ROWSUM_ALL) lsum = lsum * alpha + ((steady && STEADY_EXACT) ? e : ps[0] + ps[1]);
  };
  // alpha on the matrix accumulators; the whole wave skips it when no row's
  // reference moved (alpha == 1 everywhere, the common case)
  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        bool any = false;
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) any = any || (O_ANY && o_on_mfma(PLAN, mt, sl));
        if (any) {
          // The repurposed-MMA scaling of FlashAttention-T (section A2,
          // Fig 5(a)) in fp32: O^T <- (alpha I) O^T as 32x32x2 f32 products.
          // Slice s pairs accumulator register s of the two lane halves (rows
          // 8(s/4) + 4h + s%4, h = 0, 1) as the B operand with the matching
          // columns of alpha I as the A operand.  alpha is the same in every
          // lane here (one X = 32 tile per wave, no per-row fallback).
          f32x16 dacc = {};
#pragma unroll
          for (int sl = 0; sl < 16; ++sl) {
            if (!o_on_mfma(PLAN, mt, sl)) continue;
            const float av = (ln == 8 * (sl / 4) + 4 * hf + sl % 4) ? alpha : 0.0f;
            dacc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, oacc[mt][sl], dacc, 0, 0, 0);
          }
#pragma unroll
          for (int sl = 0; sl < 16; ++sl) oacc[mt][sl] = o_on_mfma(PLAN, mt, sl) ? dacc[sl] : oacc[mt][sl] * alpha;
          __builtin_amdgcn_sched_barrier(0);   // one tile's products at a time
        } else {
          oacc[mt] *= alpha;
        }
      }
      if constexpr (ROWSUM_ANY) lacc *= alpha;
    }
  };
  auto step_loads = [&](int j, auto XING) {
    load_k(j + kKAhead, XING);
    load_v(j + kVAhead, XING);
  };

  // Pipeline of key block b: S_b = K_b Q^T in step b-1; its tile maximum,
  // exponentials and row sums in step b, where O is rescaled by alpha_b at the
  // end (after P~_{b-1} V_{b-1}, before P~_b V_b); P~_b V_b in step b+1.

  // Any step (first, last, idle), slots and masking decided at run time.  The
  // last step (j = jend) loads nothing when the next item is prefetched: its
  // K slot holds the next item's first block.
  auto edge_step = [&](int j) {
    const unsigned long long e0 = stamp();
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
      sums_reset();
#pragma unroll
      for (int k = 0; k < 16; ++k) exp_unit(k, S[0][0], S[0][1], P[0], nb);
      sums_commit(alpha, false);
    }
    const unsigned long long e1 = stamp();
    if (j + 1 < jend_w) qk((j + 1) % kRing, S[0][0], S[0][1]);
    if (j >= 1 && j <= jend_w) pv((j - 1) % kRing, P[1]);
    const unsigned long long e2 = stamp();
    step_barrier<2 * NV_STEP>();
    if constexpr (TRACE) {
      const unsigned long long e3 = stamp();
      tr[kTrEdgeN] += 1;
      tr[kTrEdge] += e3 - e0;
      tr[kTrEdgeSoftmax] += e1 - e0;
      tr[kTrEdgeWait] += e3 - e2;
    }
    if (j < jend_w) rescale(alpha);
#pragma unroll
    for (int t = 0; t < 4; ++t) P[1][t] = P[0][t];
  };

  // Steady step j = 1 + 4g + u (u = 0..3): j >= 1 and S_j is not the wave's
  // last block.  Two phases of one straight-line block, each a run of chunks
  // of one matrix instruction and a share of the vector work on S_j:
  //   A: S_{j+1} = K_{j+1} Q^T          with the tile-maximum chain of S_j
  //                                     (computed a step ago: no wait), then
  //                                     the first EA exponential units
  //   B: O^T += V_{j-1}^T P~_{j-1}^T    with the remaining units (no
  //                                     dependency chain left to wait on)
  // The chain (d=128: parts 0-1 | 2-3 | combine | tile max | advance; d=64:
  // parts 0-3 | combine, tile max | advance) takes the first chunks of A;
  // units are spread evenly over the chunks after it and over B.  At d=128 a
  // unit's three stages go to chunks c, c+1 and c+2 of the step (clamped to
  // its last chunk), so that no stage waits for the one before it.  Operand
  // reads run LA instructions ahead; S and P~ alternate between the two
  // register sets.
  constexpr int MAXC = NQK >= 16 ? 5 : 3;      // phase-A chunks of the maximum chain
  constexpr int EA = NQK >= 16 ? 6 : 3;        // exponential units in phase A
  constexpr int LA = 3;                        // operand read lookahead
  constexpr int SKEW = NQK >= 16 ? 1 : 0;      // chunks between a unit's stages
  constexpr int LASTC = NQK + NPV - 1;         // last chunk of a step
  // chunk of unit k's first stage
  auto unit_chunk = [&](int k) -> int {
    return k < EA ? MAXC + k * (NQK - MAXC) / EA : NQK + (k - EA) * NPV / (16 - EA);
  };
  // the unit stages that fall in chunk g (in stage order for each unit)
  auto unit_stages = [&](int g, const f32x16& c0, const f32x16& c1, ev8* pk, float nb) {
    if (Z_ANY && g == MAXC) z_chain(c0, c1, nb);   // nb is known from here on
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int uc = unit_chunk(k);
      if (uc == g) unit_fma_steady(k, c0, c1, nb);
      if (min(uc + SKEW, LASTC) == g) unit_exp(k);
      if (min(uc + 2 * SKEW, LASTC) == g) unit_sum_pack(k, pk, true);
    }
  };
  auto max_chunk = [&](int i, f32x16& c0, f32x16& c1, float& alpha, float& nb) {
    if constexpr (NQK >= 16) {
      if (i == 0) { max_part(0, c0, c1); max_part(1, c0, c1); }
      if (i == 1) { max_part(2, c0, c1); max_part(3, c0, c1); }
      if (i == 2) max_combine();
      if (i == 3) tile_ref();
      if (i == 4) advance_steady(alpha, nb);
    } else {
      if (i == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) max_part(q, c0, c1);
      }
      if (i == 1) { max_combine(); tile_ref(); }
      if (i == 2) advance_steady(alpha, nb);
    }
  };
  auto steady_step = [&](auto U, int j, auto XING) {
    constexpr int u = decltype(U)::value;
    constexpr int cur = u & 1, nxt = cur ^ 1;
    const char* kt = smem + ((u + 2) % kRing) * BLK;    // K_{j+1}
    const char* vt = vring + (u % kRing) * BLK;         // V_{j-1}
    f32x16 &c0 = S[cur][0], &c1 = S[cur][1], &n0 = S[nxt][0], &n1 = S[nxt][1];
    const unsigned long long s0 = stamp();
    step_loads(j, XING);
    ev8 kop[LA], vop[LA];
#pragma unroll
    for (int g = 0; g < LA; ++g) kop[g] = kread(kt, g);
    float alpha = 1.0f, nb = 0.0f;
    sums_reset();
    // Phase A runs at raised wave priority and phase B at the default: when
    // the two waves of a SIMD are in different phases, the one still in phase
    // A (behind) is issued first, which keeps the pair in step.
    __builtin_amdgcn_s_setprio(1);
    // phase A: units 0..EA-1 start in the chunks after the chain
#pragma unroll
    for (int g = 0; g < NQK; ++g) {
      const ev8 av = kop[g % LA];
      if (g + LA < NQK) kop[g % LA] = kread(kt, g + LA);
      else vop[(g + LA - NQK) % LA] = vread(vt, g + LA - NQK);
      qk_mfma(g, av, n0, n1);
      max_chunk(g, c0, c1, alpha, nb);
      unit_stages(g, c0, c1, P[cur], nb);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    const unsigned long long s1 = stamp();
    // phase B: units EA..15 start spread over the chunks
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const ev8 av = vop[i % LA];
      if (i + LA < NPV) vop[i % LA] = vread(vt, i + LA);
      pv_mfma(i, av, P[nxt]);
      unit_stages(NQK + i, c0, c1, P[cur], nb);
      __builtin_amdgcn_sched_barrier(0);
    }
    sums_commit(alpha, true);
    pin(P[cur][0]);
    pin(P[cur][1]);
    pin(P[cur][2]);
    pin(P[cur][3]);
    pin(lexact);
    if constexpr (!ROWSUM_ALL) pin(lsum);
    const unsigned long long s2 = stamp();
    step_barrier<2 * NV_STEP>();
    if constexpr (TRACE) {
      const unsigned long long s3 = stamp();
      tr[kTrSteadyN] += 1;
      tr[kTrSteady] += s3 - s0;
      tr[kTrPhaseA] += s1 - s0;
      tr[kTrPhaseB] += s2 - s1;
      tr[kTrSteadyWait] += s3 - s2;
    }
    rescale(alpha);
  };

  // ---- epilogue of an item: l, O / l, lse (reading R-7: lse = scale*ref + ln l).
  // finish() computes them and puts this wave's O rows (32 x D) in its LDS
  // staging area: with q = r / RPB (RPB rows per 256 bytes), row r's 16-byte
  // chunk c sits at position c xor (q mod CPR), its two 8-byte halves swapped
  // when r / 16 is odd, so that the 32 lanes of each 8-byte write pass cover
  // all 64 banks.  flush() stores them, whole rows per instruction, after the
  // next item's prologue wait, so that the stores do not hold up that wait.
  constexpr int CPR = RB / 16;                  // 16-byte chunks per row
  constexpr int RPB = 256 / RB;                 // rows per 256 bytes (1 or 2)
  char* const stg = w < 4 ? smem + 2 * BLK + w * SB : smem + 2 * kRing * BLK + (w - 4) * SB;
  E* o_rows = nullptr;      // the finished item's first row of this wave (uniform)
  float* lse_rows = nullptr;
  int o_nrows = 0;          // its rows below N (uniform)
  float lse_out = 0.0f;
  auto finish = [&]() {
    float l = 0.0f;
    if constexpr (ROWSUM_ANY) l = lacc[0];
    if constexpr (!ROWSUM_ALL) l += pair_reduce(lsum, [](float x, float y) { return x + y; });
    float le = pair_reduce(lexact, [](float x, float y) { return x + y; });
    if constexpr (LEAN) le += l;
    const float inv = l > 0.0f ? a.o_scale / l : 0.0f;
    const float lse_v = le > 0.0f ? a.lse_scale * st.ref + (__logf(le) - (float)Elem16<E>::kPreLog2 * 0.69314718f)
                                  : -__builtin_inff();
    if (part) {
      // a piece of an item: its O (normalised by its own row sums) and lse go
      // to the unit's workspace slot, for the merge kernel.  O as fp16, the row
      // scaled by 2^e so that its largest magnitude lies in [2^14, 2^15)
      // (pieces.hpp); e follows lse.
      char* slot = (char*)a.ws + (size_t)unit * piece_bytes(D);
      const int r = 32 * w + ln;
      float mx = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmax_raw(mx, __builtin_fabsf(oacc[mt][i]));
      mx = pair_reduce(mx, MaxOp()) * inv;
      // mx = f 2^k with f in [0.5, 1): e = 15 - k puts mx in [2^14, 2^15)
      const int e = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
      if (qvalid) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            h4 hv;
#pragma unroll
            for (int u = 0; u < 4; ++u) hv[u] = (_Float16)__builtin_ldexpf(oacc[mt][4 * g + u] * inv, e);
            *(h4*)(slot + 2 * ((size_t)r * D + 32 * mt + 8 * g + 4 * hf)) = hv;
          }
        if (hf == 0) {
          float* tail = (float*)(slot + piece_tail(D));
          tail[r] = lse_v;
          tail[kPieceRows + r] = (float)e;
        }
      }
      o_nrows = 0;          // nothing for flush()
      lse_rows = nullptr;
      return;
    }
    // (the lane's row, opaque here: its addresses are formed here, not
    // hoisted out of the item loop to hold registers through it)
    int sr = ln;
    asm volatile("" : "+v"(sr));
    // (X = 64: wave 7's row 31 goes straight to memory; its staging bytes hold
    // the tile-maximum exchange)
    const bool direct = X == 64 && w == 7 && ln == 31;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ev4 ov;
#pragma unroll
        for (int u = 0; u < 4; ++u) ov[u] = (E)(oacc[mt][4 * g + u] * inv);
        if (!direct)
          *(ev4*)(stg + sr * RB + 16 * ((4 * mt + g) ^ ((sr / RPB) % CPR)) + 8 * (hf ^ ((sr >> 4) & 1))) = ov;
        else if (qvalid)
          *(ev4*)((E*)a.o + head + (size_t)qrow * D + 32 * mt + 8 * g + 4 * hf) = ov;
      }
    const int wq0 = q0 + 32 * w;
    o_rows = (E*)a.o + head + (size_t)wq0 * D;
    lse_rows = a.lse == nullptr ? nullptr : a.lse + (size_t)bh * N + wq0;
    o_nrows = max(0, min(32, N - wq0));
    lse_out = lse_v;
    count_tiles<X, FB_AUTO>(a, st, lane, qrow);
  };
  auto flush = [&]() {
    constexpr int RPI = 64 / CPR;   // rows per instruction
    int L = lane;
    asm volatile("" : "+v"(L));     // as in finish()
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = k * RPI + L / CPR, cc = L % CPR;
      ev8 v = *(const ev8*)(stg + r * RB + 16 * (cc ^ ((r / RPB) % CPR)));
      if ((r >> 4) & 1) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
      if (r < o_nrows && !(X == 64 && w == 7 && r == 31)) *(ev8*)(o_rows + (size_t)r * D + 8 * cc) = v;
    }
    if (lse_rows != nullptr && hf == 0 && ln < o_nrows) lse_rows[ln] = lse_out;
  };

  if constexpr (X == 64) {   // sequence numbers start at 1: clear them (the
    if (lane == 0) ((int*)xslot)[4 * w + 2] = 0;   // first barrier publishes it)
  }
  if constexpr (TRACE) {
    t_first = stamp();
    rt_first = realtime();
  }
  int it = item_of(0, gid, nwg);
  set_item(it);
  bool pref = false;   // this item's first blocks are in the rings already
  for (int round = 0;; ++round) {
    const int it_next = item_of(round + 1, gid, nwg);
    set_next(it_next);
    // ---- prologue: Q, and K_0..K_3, V_0, V_1 into the rings (unless the
    // last item's steps loaded them)
    if (!pref) {
      load_q(head, qrow, qvalid);
#pragma unroll
      for (int j = 0; j < kKAhead; ++j) load_k(j, Int<0>());
#pragma unroll
      for (int j = 0; j < kVAhead; ++j) load_v(j, Int<0>());
    }
    step_barrier<0>();
    // the same wait in a form the compiler sees: the Q fragments (plain global
    // loads) are complete from here on, so no wait for them lands in the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched
    if (round > 0) flush();   // the previous item's O and lse

    row_state_init(st, X == 1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) oacc[mt] = f32x16{};
    lsum = 0.0f;
    lacc = f32x16{};
    lexact = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) P[0][t] = P[1][t] = ev8{};
    S[0][0] = S[0][1] = S[1][0] = S[1][1] = f32x16{};
    if (jend_w > 0) qk(0, S[0][0], S[0][1]);
    // step 0 refills K_0's slot: every wave must be done reading it (the
    // stores just issued may stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // steady steps in groups of 4 (constant ring slots); only a group whose
    // loads reach past the item's last block takes the crossing loads
    int j = 0;
    edge_step(j++);
    if constexpr (!SEQ) {
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
      // two more steady steps when both qualify (j + 1 < jend_w): j is 1 mod 4
      // here, so they take the group's first two slots, and after two steps the
      // register sets are back where the edge steps expect them
      if (j + 2 < jend_w) {
        steady_step(Int<0>(), j, Int<1>());
        steady_step(Int<1>(), j + 1, Int<1>());
        j += 2;
      }
    }
    for (; j <= jend; ++j) edge_step(j);
    // the last steps' loads (zeros past the item's last block) still write
    // LDS, V slots 2 and 3 among them: let every wave's land before the O
    // staging there, the next item's loads or the end of the workgroup
    if (!pref_next) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    finish();
    if (it_next >= nunits) {
      flush();
      if constexpr (TRACE) {
        stamp();
        tr[kTrWave] = t_last - t_first;
        tr[kTrRtFirst] = rt_first;
        tr[kTrRtLast] = realtime();
        tr[kTrRealtime] = tr[kTrRtLast] - rt_first;
        if (lane == 0) {
          unsigned long long* out = a.trace + ((size_t)gid * kPWaves + w) * kTraceSlots;
#pragma unroll
          for (int i = 0; i < kTraceSlots; ++i) out[i] = tr[i];
        }
      }
      break;
    }
    pref = pref_next;
    it = it_next;
    set_item(it);
  }
}

// ---------------------------------------------------------------------------
// Merge of the pieces of each item (pieces.hpp); items of one piece wrote their
// rows directly.  For each row, with the pieces' partial (O_c, lse_c):
//   lse = m + ln sum_c exp(lse_c - m), m = max_c lse_c;  O = sum_c exp(lse_c - lse) O_c.
// A piece that held no key of the row has lse_c = -inf and weight 0 (every row
// has key 0, in the item's first piece).  Workgroup (item, p) covers rows
// [p * RPW, (p + 1) * RPW) of the item, one thread per 8 consecutive columns of
// a row, so that every load of the merge is in flight at once.
// ---------------------------------------------------------------------------
template <int D> constexpr int kMergeRowsPerWg = 256 / (D / 8);

template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_merge_h16(FwdArgs a) {
  constexpr int TPR = D / 8;                   // threads per row
  constexpr int RPW = kMergeRowsPerWg<D>;      // rows per workgroup
  constexpr int NWI = kPieceRows / RPW;        // workgroups per item
  const int it = blockIdx.x / NWI;             // item: (head, query block), heaviest first
  const int BH = a.BH, N = a.N;
  const int bh = it % BH, L = it / BH, qb = CAUSAL ? a.nqb - 1 - L : L;
  // the item's first unit: the units of the heavier levels, then this level's
  // heads before bh
  int first = 0, np = 1;
  for (int l = 0; l <= L; ++l) {
    const int q = CAUSAL ? a.nqb - 1 - l : l;
    const int p = pieces_of(qblock_blocks(q, N, CAUSAL), a.split_c);
    if (l < L) first += BH * p;
    else { first += bh * p; np = p; }
  }
  if (np <= 1) return;
  const int t = threadIdx.x, col = 8 * (t % TPR);
  const int r = (blockIdx.x % NWI) * RPW + t / TPR;
  const int row = qb * kPieceRows + r;
  if (row >= N) return;
  // the item's slots (pieces.hpp): fp16 rows scaled by 2^e, then lse and e
  const char* base = (const char*)a.ws + (size_t)first * piece_bytes(D);
  const size_t stride = (size_t)piece_bytes(D);
  auto tail = [&](int c) { return (const float*)(base + c * stride + piece_tail(D)); };
  // one pass over the pieces, online: the running maximum m of their lse and
  // the sums taken against it, rescaled when it moves (no load waits for an
  // earlier piece's, so all of them are in flight at once)
  float m = -__builtin_inff();
  float acc[8] = {};
  float sum = 0.0f;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
#pragma unroll 4
  for (int c = 0; c < np; ++c) {
    const float lc = tail(c)[r], ec = tail(c)[kPieceRows + r];
    const h8 x = *(const h8*)(base + c * stride + 2 * ((size_t)r * D + col));
    if (lc == -__builtin_inff()) continue;
    const float m_new = fmaxf(m, lc);
    const float keep = __expf(m - m_new);   // 0 while m is -inf
    const float wgt = __expf(lc - m_new);
    sum = sum * keep + wgt;
    // the row's scale 2^-e rides on its weight
    const float ws = __builtin_ldexpf(wgt, -(int)ec);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = acc[u] * keep + ws * (float)x[u];
    m = m_new;
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  typedef E ev8_t __attribute__((ext_vector_type(8)));
  ev8_t ov;
#pragma unroll
  for (int u = 0; u < 8; ++u) ov[u] = (E)(acc[u] * inv);
  *(ev8_t*)((E*)a.o + (size_t)bh * N * D + (size_t)row * D + col) = ov;
  if (a.lse != nullptr && col == 0) a.lse[(size_t)bh * N + row] = sum > 0.0f ? m + __logf(sum) : m;
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
