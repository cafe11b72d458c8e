// Shared description of the matrix-core GEMMs: operand layouts, the problem
// record (up to two K segments, up to two B operands sharing one A) and the
// work-group -> tile map.
//
// Work-group -> tile mapping: the hardware deals work-groups to the 8 XCDs of
// an MI355X round-robin (work-group w runs on XCD w % 8).  tile_coords hands
// each XCD a contiguous run of tiles and walks that run in groups of GROUP_M
// tile rows, so the tiles resident on one XCD at a time share A rows and B
// columns in that XCD's L2.
#pragma once

#include "common.hpp"

namespace tp {

enum OperandLayout {
  KMAJOR = 0,   // A stored [M, K] / B stored [N, K]: K contiguous
  MNMAJOR = 1,  // A stored [K, M] / B stored [K, N]: M or N contiguous
};

struct GemmProblem {
  int M, N;
  int nseg;                  // 1 or 2 K segments summed into one result
  int K[2];
  const uint16_t* A[2];      // [segment]
  const uint16_t* B[2][2];   // [segment][B operand]
  int64_t lda[2], ldb[2];    // leading dimensions (elements) per segment; the LDS-direct kernel
                             // requires lda[1] == lda[0] and ldb[1] == ldb[0]
};

namespace gemm {

constexpr int GROUP_M = 4;

// Tile coordinates of work-group w of the problem's launch (see the file
// comment).
__device__ __forceinline__ void tile_coords(int w, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7, x = w & 7;
  const int L = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + (w >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int inner = L - g * per_group;
  tm = first_m + inner % gsize;
  tn = inner / gsize;
}

}  // namespace gemm
}  // namespace tp
