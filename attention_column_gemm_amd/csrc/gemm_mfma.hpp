// bf16 GEMM on the gfx950 matrix cores: C = sum over segments of A_s B_s,
// fp32 accumulation, result handed to a fused epilogue.
//
// Used for every dense contraction of the shard: the column-parallel GEMM
// with its activation, the row-parallel GEMM yielding a partial, their input-
// and weight-gradient GEMMs, the QKV and output projections.
//
// Design (gfx950, 64-wide waves):
//  * 256 threads = 4 waves in a 2x2 grid; block tile BM x BN (per B operand),
//    K step 64; each wave owns a (BM/2) x (BN/2) sub-tile built from 32x32x16
//    bf16 MFMAs (v_mfma_f32_32x32x16_bf16).
//  * Both operands are staged through LDS as [rows][64] bf16 with K
//    contiguous; the 16-byte chunks of a row are XOR-swizzled by the row index
//    so that the 128-bit fragment reads and the transposed block writes hit
//    distinct banks.
//  * Global reads are raw buffer loads: lanes past a ragged tile edge point
//    their offset past the buffer's end and receive zeros, with no branches.
//    Operands whose K is the slow dimension in HBM (A stored [K,M] or B stored
//    [K,N]) are loaded as 8x8 bf16 blocks with 16-byte row reads and
//    transposed in registers before the LDS write, so every layout feeds the
//    same fragment reads.
//  * Two LDS stages: the global loads of K-tile k+1 are issued before the
//    MFMAs of tile k and written to the other stage after them; one barrier
//    per K-tile.
//  * The MFMA is issued with the B fragment as its first operand, so each
//    lane's accumulators hold four consecutive output columns of one row:
//    the epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes per lane.
//  * Up to two B operands share one A tile (SwiGLU gate and up; dWg and dWu),
//    and up to two (A, B) segments accumulate into one result
//    (dX_i = dG_i Wg_i^T + dU_i Wu_i^T).
//  * Work-group -> tile mapping: the hardware deals work-groups to the 8 XCDs
//    round-robin; the mapping hands each XCD a contiguous run of tiles and
//    walks them in groups of GROUP_M tile rows so that the tiles resident on
//    one XCD share A rows and B columns in that XCD's L2.
#pragma once

#include <type_traits>

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
  int64_t lda[2], ldb[2];    // leading dimensions (elements) per segment
};

namespace gemm {

constexpr int BK = 64;
constexpr int GROUP_M = 4;

// Element offset of 16-byte chunk `chunk` of LDS tile row `row`.  The chunk is
// XOR-swizzled with bits 0-2 and 3-5 of the row, so that any 8 consecutive
// rows (fragment reads) and any 8 rows spaced by 8 (transposed block writes)
// hit 8 different chunks.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 3);
}

// One operand of one K segment: a row-major matrix behind a buffer resource.
struct Operand {
  rsrc_t rsrc;
  uint32_t ld_bytes;  // leading dimension in bytes
  int rows;           // extent of the M (or N) dimension
  int K;              // extent of the K dimension
};

__device__ __forceinline__ Operand make_operand(const uint16_t* p, int64_t ld, int rows, int K, int layout) {
  Operand o;
  const uint32_t slow = layout == KMAJOR ? (uint32_t)rows : (uint32_t)K;
  o.rsrc = make_rsrc(p, slow * (uint32_t)ld * 2u);
  o.ld_bytes = (uint32_t)ld * 2u;
  o.rows = rows;
  o.K = K;
  return o;
}

template <int ROWS, int LAYOUT, int NT>
struct TileLoader;

// K contiguous in HBM: the tile is ROWS x 8 chunks of 16 bytes; chunk item
// tid + NT*i is (row, kc) = (item / 8, item % 8).
template <int ROWS, int NT>
struct TileLoader<ROWS, KMAJOR, NT> {
  static constexpr int PER = ROWS * (BK / 8) / NT;
  static_assert(PER * NT == ROWS * (BK / 8), "chunks must divide evenly over the threads");
  u32x4 r[PER];
  __device__ __forceinline__ void load(const Operand& op, int row0, int k0) {
    const int tid = threadIdx.x, kc = tid & 7;
    const bool kok = k0 + kc * 8 < op.K;
    const uint32_t base = (uint32_t)(row0 + (tid >> 3)) * op.ld_bytes + (uint32_t)(k0 + kc * 8) * 2u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool ok = kok && row0 + (tid >> 3) + (NT / 8) * i < op.rows;
      r[i] = buf_load16(op.rsrc, ok ? base + (uint32_t)((NT / 8) * i) * op.ld_bytes : kOOB);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int tid = threadIdx.x, kc = tid & 7;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = (tid >> 3) + (NT / 8) * i;
      *reinterpret_cast<u32x4*>(s + lds_off(row, kc)) = r[i];
    }
  }
};

// M/N contiguous in HBM: a thread loads an 8 (k) x BW (rows) block, BW = 8 or
// 4, with eight row reads of 2*BW bytes and writes it transposed as BW LDS
// rows of 16 bytes (8 k values each).  BW = 4 is used when 8-wide blocks
// would leave threads idle.
template <int ROWS, int NT>
struct TileLoader<ROWS, MNMAJOR, NT> {
  static constexpr int BW = (ROWS >= NT) ? 8 : 4;
  static constexpr int NG = ROWS / BW;               // row groups
  static constexpr int NBLK = NG * (BK / 8);         // blocks of 8 k x BW rows
  static constexpr int PER = NBLK >= NT ? NBLK / NT : 1;
  static_assert(NBLK < NT || PER * NT == NBLK, "blocks must divide evenly over the threads");
  typedef typename std::conditional<BW == 8, u32x4, u32x2>::type vec_t;
  vec_t r[PER][8];
  __device__ __forceinline__ void load(const Operand& op, int row0, int k0) {
#pragma unroll
    for (int b = 0; b < PER; ++b) {
      const int blk = threadIdx.x + NT * b;
      if (NBLK < NT && blk >= NBLK) return;
      const int mg = blk % NG, kg = blk / NG;
      const bool rok = row0 + mg * BW < op.rows;
      const int kb = k0 + kg * 8;
      const uint32_t base = (uint32_t)kb * op.ld_bytes + (uint32_t)(row0 + mg * BW) * 2u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = rok && kb + j < op.K;
        const uint32_t off = ok ? base + (uint32_t)j * op.ld_bytes : kOOB;
        if constexpr (BW == 8)
          r[b][j] = buf_load16(op.rsrc, off);
        else
          r[b][j] = __builtin_amdgcn_raw_buffer_load_b64(op.rsrc, off, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int b = 0; b < PER; ++b) {
      const int blk = threadIdx.x + NT * b;
      if (NBLK < NT && blk >= NBLK) return;
      const int mg = blk % NG, kg = blk / NG;
#pragma unroll
      for (int i = 0; i < BW; ++i) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = r[b][2 * q][i >> 1], hi = r[b][2 * q + 1][i >> 1];
          w[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int row = mg * BW + i;
        *reinterpret_cast<u32x4*>(s + lds_off(row, kg)) = w;
      }
    }
  }
};

// Tile coordinates of this work-group (see the header comment).
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int w = blockIdx.x;
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

// Block tile BM x BN computed by WGM x WGN waves, each owning a
// (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA tiles.
template <int BM, int BN, int WGM, int WGN, int AL, int BL, class Epi>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) gemm_bf16_kernel(GemmProblem p, Epi epi) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int NB = Epi::NB;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave sub-tile must hold whole 32x32 MFMA tiles");
  constexpr int STAGE = (BM + NB * BN) * BK;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  f32x16 acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][i][j][e] = 0.0f;

  TileLoader<BM, AL, NT> la;
  TileLoader<BN, BL, NT> lb[NB];
  const int nk0 = (p.K[0] + BK - 1) / BK;
  const int nk = nk0 + (p.nseg > 1 ? (p.K[1] + BK - 1) / BK : 0);
  Operand opa[2], opb[2][NB];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    opa[s] = make_operand(p.A[s], p.lda[s], p.M, p.K[s], AL);
#pragma unroll
    for (int b = 0; b < NB; ++b) opb[s][b] = make_operand(p.B[s][b], p.ldb[s], p.N, p.K[s], BL);
  }

  auto issue = [&](int kt) {
    const int s = kt < nk0 ? 0 : 1;
    const int k0 = (kt - (s ? nk0 : 0)) * BK;
    la.load(opa[s], m0, k0);
#pragma unroll
    for (int b = 0; b < NB; ++b) lb[b].load(opb[s][b], n0, k0);
  };
  auto commit = [&](int stage) {
    uint16_t* s = smem + stage * STAGE;
    la.store(s);
#pragma unroll
    for (int b = 0; b < NB; ++b) lb[b].store(s + BM * BK + b * BN * BK);
  };

  if (nk > 0) {
    issue(0);
    commit(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) issue(kt + 1);
    const uint16_t* As = smem + stage * STAGE;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 af[TM], bfr[NB][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * WM + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[b][j] = *reinterpret_cast<const bf16x8*>(Bs + b * BN * BK + lds_off(wn * WN + j * 32 + (lane & 31), chunk));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b][j], af[i], acc[b][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) commit(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds, for tile (i, j), row m = .. + (lane & 31) and columns
  // n = .. + 8*q4 + 4*(lane >> 5) + e, e = 0..3, in accumulator slots 4*q4 + e.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = n0 + wn * WN + j * 32 + q4 * 8 + (lane >> 5) * 4;
        float v[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) v[b][e] = acc[b][i][j][q4 * 4 + e];
        epi(m, n, v);
      }
    }
  }
}

}  // namespace gemm

// Host-side launcher: grid of ceil(M/BM) * ceil(N/BN) work-groups of
// 64 * WGM * WGN threads.
template <int BM, int BN, int WGM, int WGN, int AL, int BL, class Epi>
hipError_t launch_gemm_bf16(const GemmProblem& p, const Epi& epi, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm::gemm_bf16_kernel<BM, BN, WGM, WGN, AL, BL, Epi>), dim3(tiles), dim3(64 * WGM * WGN), 0,
                     stream, p, epi);
  return hipGetLastError();
}

}  // namespace tp
