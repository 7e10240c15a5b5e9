// Workgroup-to-work maps of the large launches, shared by the kernels and
// by the measurement kernels that mirror their grids.  Workgroups are dealt
// round-robin to the eight dies (XCDs) of an MI355X, each with its own L2;
// these maps only decide which die does which part of the work, never what
// is computed.
#pragma once

#include <hip/hip_runtime.h>

namespace isb {

constexpr int kScoreWaves = 4;        // waves (blocks) per workgroup of the index scan

// Column group of request r taken by workgroup column p of gx, for workgroups
// of BPW blocks.  Workgroups are dealt round-robin to the eight dies (XCDs),
// each with its own L2.  This mapping hands each die whole 32-block spans (one
// 128-byte line of a score row), so the workgroups that write a line share an
// L2, which merges their 4- and 8-byte writes before the line goes to HBM
// (spread over eight L2s, each partial line was written back on its own).
// The spans rotate over the dies from request to request: the spans past a
// short request's end hold no keys, and a fixed span-to-die map would leave
// the dies that own the last spans idle.  Any mapping is correct; this one
// only places the work.
template <int BPW>
__device__ __forceinline__ int score_column(int p, int gx, int r) {
  constexpr int LW = 32 / BPW;  // workgroups per span
  const int full = gx / (8 * LW) * (8 * LW);
  if (p >= full) return p;
  const int k = p & 7, q = p >> 3;
  const int j = q / LW, w = q % LW;
  return LW * (8 * j + ((k + r) & 7)) + w;
}

// Row of grid column x.  Workgroups are dealt round-robin to the eight dies
// (XCDs), each with its own L2; consecutive rows (the tokens of one request,
// whose selections share blocks) are given to one die, die d taking rows
// [d R / 8, (d + 1) R / 8), so a block several of them attend is fetched into
// that die's L2 once.  A permutation of the rows: any mapping gives the same
// results.  Rows past the last multiple of eight keep their column.
__device__ __forceinline__ int grid_row(int x, int rows) {
  const int per = rows >> 3;
  return x < 8 * per ? (x & 7) * per + (x >> 3) : x;
}

}  // namespace isb
