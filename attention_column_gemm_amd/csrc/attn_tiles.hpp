// LDS tile helpers shared by the attention kernels: a row-major [rows][D]
// bf16 tile with a 16-byte-chunk swizzle, its 128-bit row fragments, its
// transposed fragments read with ds_read_b64_tr_b16, and the LDS-direct
// loader that fills it.
#pragma once

#include "common.hpp"
#include "lds_dma.hpp"

namespace tp {
namespace attnt {

using lds::lds_u8;
using lds::v4i16;

// Query block and head-group index of this work-group in a causal launch of
// an npb x ny grid (query blocks x head groups) whose work-groups are all
// resident at once, two per CU.  A later query block sees more keys, so the
// blocks are ranked by work, heaviest first; the first half of the dispatch
// order takes ranks 0, 1, 2, ... and the second half takes them from the
// lightest back up, so that the work-group that fills a CU's second slot is
// light where the first was heavy.  Dispatch order is blockIdx.x fastest.
__device__ __forceinline__ void causal_block_order(int npb, int ny, int& pb, int& y) {
  const int total = npb * ny;
  const int L = (int)blockIdx.x + (int)blockIdx.y * npb;
  const int half = (total + 1) / 2;
  const int r = L < half ? L : total - 1 - (L - half);
  pb = npb - 1 - r / ny;
  y = r % ny;
}

// 16-byte chunk permutation of a row-major [rows][D] bf16 tile: logical chunk
// c of row r sits at chunk c ^ swz(r).  Two reads must both be conflict-free
// on gfx950's 64 banks of 4 bytes: 128-bit row fragments (16 lanes per pass,
// 16 consecutive rows, one chunk each) and transposing reads (32 lanes per
// pass, four consecutive rows, four chunks each).  D = 128 (256-byte rows, each starting on the same
// bank): the low two row bits pick one of four groups of four chunks and the
// next two the chunk within the group.  D = 64 (128-byte rows, even and odd
// rows in opposite bank halves): row bit 1 picks the group, bits 2-3 the chunk.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ uint32_t tile_off(int r, int c) {
  return (uint32_t)(r * D * 2 + ((c ^ swz<D>(r)) << 4));
}

// 16-byte row fragment (rows r0 + lane%32, k step kk) of a row-major tile.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const lds_u8* tile, int r0, int kk) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
      tile + tile_off<D>(r0 + (lane & 31), kk * 2 + (lane >> 5)));
}

// Transposed fragment of a row-major tile T[row][col]: lane l gets column
// 32 dt + l % 32 at the eight rows that the registers 8 jj .. 8 jj + 7 of a
// 32x32 accumulator hold for its half h = l / 32, i.e. rows
// r0 + 16 jj + 4 h + {0..3} and r0 + 16 jj + 8 + 4 h + {0..3}.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const lds_u8* tile, int r0, int dt, int jj) {
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, R = lane & 15, h = lane >> 5;
  const int col = 32 * dt + 16 * (g4 & 1) + 4 * (R & 3);
  v4i16 part[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = r0 + 16 * jj + 4 * h + 8 * half + (R >> 2);
    part[half] = lds::read_tr16(tile, tile_off<D>(row, col >> 3) + (col & 7) * 2);
  }
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

// LDS-direct load of rows [row0, row0 + ROWS) x D bf16 columns starting at
// byte column col_bytes of a row-major matrix (ld_bytes per row, nrows rows,
// behind `rsrc`) into a swizzled [ROWS][D] tile at LDS byte address dst:
// instruction i of the tile's ROWS * D * 2 / 1024 one-KiB instructions.
// Row offsets use the full-rate 24-bit multiply: row indices and ld_bytes
// stay below 2^24 (the host rejects larger attention shapes).
template <int D>
__device__ __forceinline__ void dma_tile_part(const u32x4& rsrc, uint32_t ld_bytes, int row0, int nrows,
                                              uint32_t col_bytes, uint32_t dst, int i) {
  const int lane = threadIdx.x & 63;
  const int o = i * 1024 + 16 * lane;
  const int r = o / (2 * D), pos = (o % (2 * D)) >> 4;
  const int c = pos ^ swz<D>(r);
  const uint32_t voff =
      row0 + r < nrows ? __umul24((uint32_t)(row0 + r), ld_bytes) + col_bytes + (uint32_t)c * 16u : kOOB;
  lds::dma16(rsrc, voff, dst + (uint32_t)i * 1024u);
}

// The same load with the per-lane half of the source offset computed once:
// dma_lane_off<D>(ld_bytes, i0) serves every instruction i that swz<D>
// cannot tell apart from i0 (it sees rows modulo 16, and instruction i
// starts at row RI i: i = i0 mod 4 for D = 128, mod 2 for D = 64), and
// the rest of the offset is wave-uniform.  Rows at or past the
// descriptor's end (num_records = nrows ld_bytes) read zeros.
template <int D>
__device__ __forceinline__ uint32_t dma_lane_off(uint32_t ld_bytes, int i0) {
  constexpr int CPR = 2 * D / 16, RI = 1024 / (2 * D);  // 16-byte chunks per row, rows per instruction
  const int lane = threadIdx.x & 63;
  const int rl = lane / CPR;
  const int c = (lane % CPR) ^ swz<D>(i0 * RI + rl);
  return __umul24((uint32_t)rl, ld_bytes) + (uint32_t)c * 16u;
}
template <int D>
__device__ __forceinline__ void dma_tile_part_at(const u32x4& rsrc, uint32_t ld_bytes, int row0, uint32_t col_bytes,
                                                 uint32_t dst, int i, uint32_t lane_off) {
  constexpr int RI = 1024 / (2 * D);
  lds::dma16(rsrc, lane_off + (uint32_t)(row0 + i * RI) * ld_bytes + col_bytes, dst + (uint32_t)i * 1024u);
}

// The whole tile: this wave issues instructions i0, i0 + step, ...
template <int D, int ROWS>
__device__ __forceinline__ void dma_tile(const u32x4& rsrc, uint32_t ld_bytes, int row0, int nrows,
                                         uint32_t col_bytes, uint32_t dst, int i0, int step) {
  constexpr int NI = ROWS * D * 2 / 1024;
  for (int i = i0; i < NI; i += step) dma_tile_part<D>(rsrc, ld_bytes, row0, nrows, col_bytes, dst, i);
}

// One 4-byte load per lane from `rsrc` at `voff` into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(const u32x4& rsrc, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rsrc)
               : "memory");
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

}  // namespace attnt
}  // namespace tp
