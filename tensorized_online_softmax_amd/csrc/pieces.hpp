// pieces.hpp -- work units of the persistent 16-bit kernel when a problem has
// fewer query blocks than compute units: each item (a 256-row query block of a
// head) is cut into pieces of at most C key blocks, so that every compute unit
// gets work.  Each piece runs the online softmax over its own key range and
// leaves a partial result (O normalised by its own row sums, and its lse); a
// second kernel merges the pieces of an item exactly:
//   lse = ln sum_c exp(lse_c),   O = sum_c exp(lse_c - lse) O_c,
// the same rescale by exp(m_old - m) that the online softmax applies block by
// block (FlashAttention-T, section A3, Fig 2(a)), here between key ranges.
// Shared by the host (sizes) and the kernels (unit -> piece, the slot layout).
#pragma once
#include <hip/hip_runtime.h>

namespace tos {

constexpr int kPieceRows = 256;        // query rows of an item (the kernel's workgroup)
constexpr int kPieceBc = 64;           // keys per block
constexpr int kMaxPieces = 256;        // at most this many units when pieces are cut
constexpr int kMinPieceBlocks = 8;     // shortest piece worth its prologue and epilogue

// key blocks of query block qb of a head: all of them, or (causal) up to its last row
__host__ __device__ inline int qblock_blocks(int qb, int N, bool causal) {
  const int nblk = (N + kPieceBc - 1) / kPieceBc;
  if (!causal) return nblk;
  const int last = min((qb + 1) * kPieceRows, N) - 1;
  return last / kPieceBc + 1;
}

__host__ __device__ inline int pieces_of(int nblocks, int C) { return C > 0 ? (nblocks + C - 1) / C : 1; }

struct Piece {
  int bh, qb;      // head and query block (the item)
  int jb, je;      // its key blocks [jb, je)
  int first, np;   // the item's first unit and its number of pieces
};

// Unit u of a launch over BH heads of nqb query blocks.  Items are numbered
// heaviest first (causal: the query blocks with the most keys), heads fastest;
// with C > 0 the pieces of an item are consecutive units and split its key
// blocks as evenly as they go.
__host__ __device__ inline Piece piece_of(int u, int BH, int nqb, int N, bool causal, int C) {
  Piece p{};
  if (C <= 0) {
    p.bh = u % BH;
    p.qb = causal ? nqb - 1 - u / BH : u / BH;
    p.jb = 0;
    p.je = qblock_blocks(p.qb, N, causal);
    p.first = u;
    p.np = 1;
    return p;
  }
  int base = 0;
  for (int L = 0; L < nqb; ++L) {
    const int qb = causal ? nqb - 1 - L : L;
    const int n = qblock_blocks(qb, N, causal);
    const int np = pieces_of(n, C);
    if (u < base + BH * np) {
      const int r = u - base, c = r % np;
      p.bh = r / np;
      p.qb = qb;
      p.jb = (int)((long long)c * n / np);
      p.je = (int)((long long)(c + 1) * n / np);
      p.first = base + p.bh * np;
      p.np = np;
      return p;
    }
    base += BH * np;
  }
  return p;   // u out of range: an empty piece
}

// number of units over all items with pieces of at most C blocks (C = 0: items)
__host__ __device__ inline long long units_of(int BH, int nqb, int N, bool causal, int C) {
  long long u = 0;
  for (int qb = 0; qb < nqb; ++qb) u += (long long)BH * pieces_of(qblock_blocks(qb, N, causal), C);
  return u;
}

// Workspace per unit, in bytes: the partial O as fp16 (256 rows x d), each row
// scaled by 2^e so that its largest magnitude lies in [2^14, 2^15) -- fp16's
// 11 bits relative to the row's largest value, whatever the range of V --
// then per row its lse (256 floats) and its e (256 floats).
__host__ __device__ constexpr long long piece_bytes(int d) { return (long long)kPieceRows * (2 * d + 8); }
// byte offset, within a unit's slot, of its 256 lse values (the e values follow)
__host__ __device__ constexpr long long piece_tail(int d) { return (long long)kPieceRows * 2 * d; }

}  // namespace tos
