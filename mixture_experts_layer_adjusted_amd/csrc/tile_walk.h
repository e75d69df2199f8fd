// Index math of the grouped GEMMs' tile order, shared by the device kernels and a host checker.
//
// The permutation lays every segment (one routed expert's tokens in increasing order, then one
// full-token segment per shared expert) out from a multiple of 128 rows; the grouped GEMMs cut
// each segment into M-tiles of TM rows (128, or 256 = a pair of 128-row tiles, the last one of a
// segment with an odd count being a half tile) and the output features into NT tiles.  Logical
// tile l lies in the segment owning its M-tile slot l / NT; within a segment the tiles are dealt
// in blocks of group_m M-tiles x NT N-tiles, M fastest, so that the 32 workgroups an XCD holds
// share both operands' slices in its L2.  Workgroup b of a one-tile grid runs on XCD b mod 8 and
// takes logical tile xcd_logical(b); a persistent workgroup b of G walks persistent_first(b, G),
// + G, + 2G, ... (the same XCD throughout).
//
// Everything here is plain integer arithmetic on values the caller has read from the segment
// tables, so the same functions run in the kernels and in the CPU bounds check.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif

namespace moe {

constexpr int kWalkTileM = 128;     // rows of an M-tile; segments start on multiples of it
constexpr int kWalkXcds = 8;        // XCDs of MI355X; workgroups are dealt to them round-robin
constexpr int kWalkXcdChunk = 32;   // workgroups an XCD holds at once (one per CU)

MOE_HD int walk_imin(int a, int b) { return a < b ? a : b; }

// Workspace bound on the M-tiles of any routing of T tokens to K of n_routed experts: the routed
// loads sum to T K, so the sum over experts of ceil(load / 128) is at most (T K + 127 n_routed) / 128;
// each shared expert adds ceil(T / 128).
MOE_HD int64_t walk_max_tiles(int64_t T, int64_t K, int64_t n_routed, int64_t n_shared) {
  return (T * K + n_routed * (kWalkTileM - 1)) / kWalkTileM + n_shared * ((T + kWalkTileM - 1) / kWalkTileM);
}

// Bound on the 256-row tiles: a segment of c M-tiles has ceil(c / 2) <= (c + 1) / 2 of them, so
// n_seg segments have at most (max_tiles + n_seg) / 2, and never more than max_tiles.
MOE_HD int64_t walk_max_pairs(int64_t max_tiles, int64_t n_seg) {
  const int64_t b = (max_tiles + n_seg) / 2;
  return b < max_tiles ? b : max_tiles;
}

// logical tile of workgroup b in a one-tile grid (blocks of kWalkXcds * chunk workgroups; inside a
// block, the `chunk` workgroups one XCD holds at once take consecutive logical tiles)
MOE_HD int64_t xcd_logical(int64_t b, int chunk = kWalkXcdChunk) {
  const int64_t span = (int64_t)kWalkXcds * chunk;
  return (b / span) * span + (b % kWalkXcds) * chunk + (b / kWalkXcds) % chunk;
}

// first logical tile of persistent workgroup b of G (G a multiple of kWalkXcds); it then steps by G
MOE_HD int persistent_first(int b, int G) { return (b % kWalkXcds) * (G / kWalkXcds) + b / kWalkXcds; }

struct WalkTile {
  int nt;          // N-tile
  int tile_rows;   // rows of the M-tile inside its segment (TM, or 128 for the half tile of a pair walk)
  int64_t m0;      // first row of the M-tile in the permuted layout
};

// The tile of logical index l in segment seg, given that segment's first M-tile slot (seg_first),
// its number of slots (seg_count), and its rows [row_start, row_end) in the permuted layout
// (row_end = the next segment's start: padding rows included).
MOE_HD WalkTile walk_tile(int64_t l, int NT, int group_m, int TM, int seg_first, int seg_count, int row_start,
                          int row_end) {
  const int64_t lam = l - (int64_t)seg_first * NT;
  const int grp = (int)(lam / ((int64_t)group_m * NT));
  const int gm = walk_imin(group_m, seg_count - grp * group_m);
  const int rem = (int)(lam - (int64_t)grp * group_m * NT);
  const int local = grp * group_m + rem % gm;
  WalkTile t;
  t.nt = rem / gm;
  t.m0 = (int64_t)row_start + (int64_t)local * TM;
  t.tile_rows = walk_imin(TM, row_end - (int)t.m0);
  return t;
}

}  // namespace moe
