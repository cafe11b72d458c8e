// bf16 GEMM on the gfx950 matrix cores with LDS-direct loads and a
// two-stage K pipeline: C = sum over segments of A_s B_s, fp32 accumulation,
// result handed to a fused epilogue (same problem description and epilogues
// as gemm_common.hpp).
//
// Why this shape (gfx950):
//  * Operand tiles go from HBM straight into LDS with 16-byte buffer loads
//    that write LDS ("buffer_load_dwordx4 ... lds"): no staging registers,
//    no ds_write instructions, and ragged edges read zeros because their
//    offsets point past the buffer resource's end.
//  * K advances in tiles of BK = 64 through two LDS stages; the loads of tile
//    t+1 are in flight while tile t is consumed.  One barrier per tile, placed
//    before the tile's last 16-deep k step so that the next tile's first
//    fragments are read from LDS while that step's MFMAs execute.  BK = 64
//    with two stages measured faster than BK = 32 with three or four (fewer
//    barriers), and an explicit L2 warm-up of the tile after next did not
//    help.
//  * The waves split into two halves, one wave of each on every SIMD; the
//    halves issue their share of a tile's loads one or two k steps apart, so
//    that on every SIMD one wave can issue MFMAs while the other is handing
//    loads to the memory pipeline (measured 3-7% over issuing all loads at
//    once).  The last K tile is peeled off the loop, scheduling groups
//    spread each k step's fragment reads over its MFMAs, and with both
//    operands K-contiguous each half runs its own copy of the loop (see the
//    loop).  Taking the LDS-direct loads out of the loop (a measurement
//    switch) speeds it up by about a quarter; they are what limits it.
//  * K-contiguous operands live in LDS as [rows][BK] with the 16-byte chunks
//    of a row XOR-swizzled by the row index (conflict-free 128-bit fragment
//    reads).  M/N-contiguous operands (weights stored [K,N], the
//    transposed activations of the weight gradients) live as [BK][rows] with
//    their 16-byte chunks swizzled by k, and are read into the MFMA's
//    K-contiguous register layout with ds_read_b64_tr_b16 (gfx950's
//    transposing LDS read): no transposition ever goes through registers.
//  * v_mfma_f32_32x32x16_bf16 with the B fragment as first operand, so a
//    lane's accumulators are four consecutive output columns (8- or 16-byte
//    stores).  Accumulators stay in arch VGPRs (the AGPR form measured slower).
//  * The blockIdx -> tile map is the XCD-aware grouped map of gemm_common.hpp.
//  * Launch shapes around the tile body: one problem per launch; two
//    independent problems in one launch (gemm_dma_pair_kernel), so each
//    fills the CUs the other's last round leaves idle; and a split tail
//    (SplitTail), where the tiles of a last round at most half full each run
//    as two K halves whose fp32 partials a second kernel adds.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"
#include "lds_dma.hpp"

namespace tp {
namespace gemm3 {

using lds::lds_u8;
using lds::v4i16;
using lds::sgpr_rsrc;
using lds::dma16;
using lds::wait_vmcnt;
using lds::barrier;

// Byte offset of 16-byte chunk c of row `row` in a K-contiguous [ROWS][32] tile.
// Rows of BK = 32 are 64 bytes (4 chunks, swizzled by row bits 2-3); rows of
// BK = 64 are 128 bytes (8 chunks, swizzled by row bits 0-2 xor 3-5).  Either
// way 16 consecutive rows at one logical chunk hit 16 distinct bank groups.
template <int BK>
__device__ __forceinline__ uint32_t kofs(int row, int c) {
  if (BK == 32) return row * 64 + ((c ^ ((row >> 2) & 3)) << 4);
  return row * 128 + ((c ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// XOR applied to the 16-byte chunk index within k-row k of an M/N-contiguous
// tile of NCH chunks per k-row.  A transposing fragment read serves 32 lanes
// per pass from four consecutive k-rows (k = 4j .. 4j+3) and four chunks of
// each; with 64 banks of 4 bytes, k-rows of 256 or 512 bytes start on the
// same bank, so those four k-rows must land in four different groups of four
// chunks: XOR with 4 (k & 3).  k-rows of 128 bytes alternate between the two
// bank halves by themselves, and XOR with 2 (k & 7) keeps them apart.
template <int NCH>
__device__ __forceinline__ int mswz(int k) {
  if constexpr (NCH >= 16)
    return ((k & 3) << 2) & (NCH - 1);
  else
    return ((k & 7) << 1) & (NCH - 1);
}

// Byte offset of 16-byte chunk c of k-row k in an M/N-contiguous [BK][ROWS] tile.
template <int ROWS>
__device__ __forceinline__ uint32_t mofs(int k, int c) {
  constexpr int NCH = ROWS / 8;
  return k * ROWS * 2 + ((c ^ mswz<NCH>(k)) << 4);
}

struct DOperand {
  u32x4 rsrc;
  uint32_t ld_bytes;
  int rows, K;
};

__device__ __forceinline__ DOperand make_doperand(const uint16_t* p, int64_t ld, int rows, int K, int layout) {
  DOperand o;
  const uint32_t slow = layout == KMAJOR ? (uint32_t)rows : (uint32_t)K;
  o.rsrc = sgpr_rsrc(p, slow * (uint32_t)ld * 2u);
  o.ld_bytes = (uint32_t)ld * 2u;
  o.rows = rows;
  o.K = K;
  return o;
}

// Per-lane source coordinates of the LDS-direct loads of one operand tile.
// The tile is ROWS * 64 bytes = ROWS/16 wave-instructions of 1 KiB; wave w
// issues instructions w*PER .. w*PER+PER-1, lane l fills LDS chunk
// q = instr*64 + l.
template <int ROWS, int LAYOUT, int NW, int BK>
struct DmaLoader {
  static constexpr int INSTR = ROWS * BK * 2 / 1024;
  static constexpr int PER = INSTR / NW;
  static_assert(PER >= 1 && PER * NW == INSTR, "tile instructions must divide evenly over the waves");
  uint32_t base[PER];  // byte offset of this lane's chunk for k0 = 0
  int kloc[PER];       // k index of the chunk within the tile; 2^30 if its M/N row is outside the matrix
  uint32_t m0off;      // this wave's first LDS destination within a tile (bytes)

  // row0: first M/N row of the tile; ld_bytes, rows: the operand's leading
  // dimension and M/N extent (the same for every K segment).
  __device__ __forceinline__ void init(int row0, uint32_t ld_bytes, int rows) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, so m0 stays scalar
    m0off = (uint32_t)(wave * PER) * 1024u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = (wave * PER + i) * 64 + lane;
      int r, k;
      if (LAYOUT == KMAJOR && BK == 32) {
        const int row = q >> 2, p = q & 3;
        r = row;
        k = (p ^ ((row >> 2) & 3)) * 8;
      } else if (LAYOUT == KMAJOR) {
        const int row = q >> 3, p = q & 7;
        r = row;
        k = (p ^ ((row ^ (row >> 3)) & 7)) * 8;
      } else {
        constexpr int NCH = ROWS / 8;
        const int kk = q / NCH, p = q % NCH;
        k = kk;
        r = (p ^ mswz<NCH>(kk)) * 8;
      }
      r += row0;
      kloc[i] = r < rows ? k : (1 << 30);
      base[i] = LAYOUT == KMAJOR ? (uint32_t)r * ld_bytes + (uint32_t)k * 2u : (uint32_t)k * ld_bytes + (uint32_t)r * 2u;
    }
  }
  // Loads of the K tile starting at k0 into the LDS tile at lds_tile.
  __device__ __forceinline__ void issue(const DOperand& op, int k0, uint32_t lds_tile) const {
    const uint32_t kbytes = LAYOUT == KMAJOR ? (uint32_t)k0 * 2u : (uint32_t)k0 * op.ld_bytes;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dma16(op.rsrc, kloc[i] + k0 < op.K ? base[i] + kbytes : kOOB, lds_tile + m0off + (uint32_t)i * 1024u);
    }
  }
};

// MFMA operand fragment (32 rows x 16 k) of the tile row block starting at
// `tr`, k step kk (0 .. BK/16-1), from an LDS tile of the given layout.
template <int ROWS, int LAYOUT, int BK>
__device__ __forceinline__ bf16x8 fragment(const lds_u8* tile, int tr, int kk) {
  const int lane = threadIdx.x & 63;
  if (LAYOUT == KMAJOR) {
    const int row = tr + (lane & 31), c = kk * 2 + (lane >> 5);
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + kofs<BK>(row, c));
  } else {
    // ds_read_b64_tr_b16: within each 16-lane group, lane R supplies the
    // address of 4 consecutive rows at k-row kb + R/4, rows m_base + 4*(R%4);
    // lane i then holds rows m_base + i at k = kb .. kb+3.
    const int g = lane >> 4, R = lane & 15;
    const int m = tr + 16 * (g & 1) + 4 * (R & 3);
    v4i16 h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = kk * 16 + 8 * (g >> 1) + 4 * half + (R >> 2);
      const uint32_t off = mofs<ROWS>(k, m >> 3) + (m & 7) * 2;
      h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_u8*>(tile) + off));
    }
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  }
}

// Scheduling groups for one k step of NMF MFMAs and NDS LDS fragment reads:
// read group I (sized to spread NDS reads over the first NMF-2 slots), then
// MFMA I.
template <int I, int NMF, int NDS>
__device__ __forceinline__ void interleave_reads() {
  if constexpr (I < NMF) {
    constexpr int SLOTS = NMF - 2;
    constexpr int r = I < SLOTS ? ((I + 1) * NDS + SLOTS - 1) / SLOTS - (I * NDS + SLOTS - 1) / SLOTS : 0;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // one MFMA
    interleave_reads<I + 1, NMF, NDS>();
  }
}

// Operand stages in LDS: two for the 256- and 128-row tiles; the 64 x 64
// tile, whose waves issue one MFMA per k step and so cannot cover a K tile's
// load latency with one tile in flight, takes three (two tiles in flight
// while one is read; measured on gfx950 against two and four stages).
template <int BM, int BN, int NB>
constexpr int gemm_nstage() {
  return BM * BN <= 64 * 64 ? 3 : 2;
}
// LDS bytes of one work-group: the operand stages, reused by the epilogue's
// staging area once the K loop is done.
template <int BM, int BN, int WGM, int WGN, int BK, int NB>
constexpr int smem_bytes() {
  constexpr int STAGE = BM * BK * 2 + NB * BN * BK * 2;
  constexpr int STAGES = gemm_nstage<BM, BN, NB>() * STAGE;
  constexpr int STAGING = WGM * WGN * NB * 32 * ((BN / WGN) * 4 + 16);  // epilogue staging (see below)
  return STAGES > STAGING ? STAGES : STAGING;
}

// One output tile: tile w of problem p's launch, computed by the whole
// work-group with `smem` (smem_bytes() bytes, 1 KiB aligned) as its LDS.
// With KRANGE the K tiles kt_begin .. kt_begin + n_kt - 1 are accumulated
// (the K tiles of the segments numbered consecutively), otherwise all of them.
// With rows_win > 0, w numbers the tiles of the tile rows tm_lo ..
// tm_lo + rows_win - 1 only (the same XCD-aware order within that window).
template <int BM, int BN, int WGM, int WGN, int BK, int AL, int BL, class Epi, bool KRANGE = false>
__device__ __forceinline__ void gemm_dma_tile(const GemmProblem& p, const Epi& epi, int w, uint8_t* smem,
                                              int kt_begin = 0, int n_kt = 0, int tm_lo = 0, int rows_win = 0) {
  constexpr int NW = WGM * WGN;
  constexpr int NB = Epi::NB;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave sub-tile must hold whole 32x32 MFMA tiles");
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + NB * B_BYTES;
  constexpr int NSTAGE = gemm_nstage<BM, BN, NB>(), KK = BK / 16;
  static_assert(KK >= 3 && NW % 2 == 0, "staggered issue needs at least three k steps and paired waves");

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  gemm::tile_coords(w, rows_win > 0 ? rows_win : tiles_m, tiles_n, tm, tn);
  tm += tm_lo;
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const lds_u8* lds = (const lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  f32x16 acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][i][j][e] = 0.0f;

  DmaLoader<BM, AL, NW, BK> la;
  DmaLoader<BN, BL, NW, BK> lb;
  // every K segment shares the leading dimensions of segment 0 (host contract)
  la.init(m0, (uint32_t)p.lda[0] * 2u, p.M);
  lb.init(n0, (uint32_t)p.ldb[0] * 2u, p.N);

  const int nk0 = (p.K[0] + BK - 1) / BK;
  const int nk_all = nk0 + (p.nseg > 1 ? (p.K[1] + BK - 1) / BK : 0);
  const int nk = KRANGE ? n_kt : nk_all;  // K tiles of this work-group, counted from kt_begin
  DOperand opa[2], opb[2][NB];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    opa[s] = make_doperand(p.A[s], p.lda[s], p.M, p.K[s], AL);
#pragma unroll
    for (int b = 0; b < NB; ++b) opb[s][b] = make_doperand(p.B[s][b], p.ldb[s], p.N, p.K[s], BL);
  }

  // With a K-contiguous A and a single M/N-contiguous B the waves issue their
  // LDS-direct loads at raised priority, ahead of the SIMD's other wave
  constexpr bool PRIO_LOADS = AL == KMAJOR && BL != KMAJOR && NB == 1;
  // kt (local) may lie past the last tile (by one with two stages, by up to
  // NSTAGE with the deeper pipeline): it is then sent past the end of K,
  // where every offset is out of range and the loads only write zeros into
  // LDS
  auto issue = [&](int kt) {
    const int gk = KRANGE ? (kt < nk ? kt_begin + kt : nk_all) : kt;
    const int s = (gk < nk0 || p.nseg == 1) ? 0 : 1;
    const int k0 = (gk - (s ? nk0 : 0)) * BK;
    const uint32_t st = lds_base + (uint32_t)(kt % NSTAGE) * STAGE;
    if constexpr (PRIO_LOADS) __builtin_amdgcn_s_setprio(2);
    la.issue(opa[s], k0, st);
#pragma unroll
    for (int b = 0; b < NB; ++b) lb.issue(opb[s][b], k0, st + A_BYTES + b * B_BYTES);
    if constexpr (PRIO_LOADS) __builtin_amdgcn_s_setprio(0);
  };

  // Fragments of one k step (16 of the tile's 32 k) for all of this wave's MFMA tiles.
  struct Frags {
    bf16x8 a[TM], b[NB][TN];
  };
  auto load_frags = [&](Frags& F, int kt, int kk) {
    const lds_u8* As = lds + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i) F.a[i] = fragment<BM, AL, BK>(As, wm * WM + i * 32, kk);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < TN; ++j) F.b[b][j] = fragment<BN, BL, BK>(As + A_BYTES + b * B_BYTES, wn * WN + j * 32, kk);
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.b[b][j], F.a[i], acc[b][i][j], 0, 0, 0);
  };
  // Waves 0 .. NW/2-1 form half 0, the rest half 1; wave w runs on SIMD w % 4,
  // so with eight waves every SIMD holds one wave of each half.  Half 0
  // issues its share of tile t+1 right after the barrier that frees the
  // stage (one k step before tile t starts), half 1 at k step STAGGER of tile
  // t: step 0, except step 1 for the large single-B tile with M-contiguous A
  // (the weight gradients' transposing fragment reads keep its LDS busier);
  // measured on gfx950, later points leave the loads too little time to
  // land.  Each wave waits for its own loads (vmcnt 0) before the next
  // barrier.
  constexpr int STAGGER = (AL != KMAJOR && NB == 1 && BM == 256) ? 1 : 0;
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / (NW / 2);
  auto sync_next = [&]() {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    barrier();
  };
  Frags F[2];
  // Scheduling hint for one k step: the next step's fragment reads are
  // spread over all but the last two of this step's MFMAs instead of being
  // bunched, so no MFMA waits on a read issued just before it (measured 1-5%
  // on gfx950).  With an M-contiguous B and a K-contiguous A the hint makes
  // the compiler spill and is left out.
  auto interleave = [&]() {
    if constexpr (!(AL == KMAJOR && BL != KMAJOR && NB == 1)) {
      constexpr int NMF = NB * TM * TN;
      constexpr int NDS = TM * (AL == KMAJOR ? 1 : 2) + NB * TN * (BL == KMAJOR ? 1 : 2);
      interleave_reads<0, NMF, NDS>();
    }
  };
  if (NSTAGE == 2 && nk > 0) {
    issue(0);
    sync_next();
    if (half == 0 && nk > 1) issue(1);
    load_frags(F[0], 0, 0);
  }
  // All K tiles but the last.  The last one is peeled off so that the step
  // after each barrier has a single predecessor: its MFMAs then consume
  // fragments already complete at the barrier without waiting for the next
  // tile's first reads.  With both operands K-contiguous each half of the
  // waves runs its own copy of the loop, in which its loads sit at a fixed
  // step with no branch around them, so the compiler schedules every k step
  // as one block (3-5% on gfx950; the other layouts spill with two copies).
  // Half 0's refill on the loop's last pass targets tile nk and only writes
  // zeros into the stage that has just been freed.
  // H: 0 or 1 for a copy specialised to that half, 2 for the shared copy
  auto kloop = [&](auto half_c) {
    constexpr int H = decltype(half_c)::value;
    for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          if (kk == STAGGER && (H == 1 || (H == 2 && half == 1))) issue(kt + 1);
          load_frags(F[(kk + 1) & 1], kt, kk + 1);
        } else {
          // tile kt+1 has landed and every read of tile kt's stage is done, so
          // half 0 may refill it with tile kt+2
          sync_next();
          if (H == 0 || (H == 2 && half == 0 && kt + 2 < nk)) issue(kt + 2);
          load_frags(F[(kk + 1) & 1], kt + 1, 0);
        }
        mfmas(F[kk & 1]);
        interleave();
      }
    }
  };
  if constexpr (NSTAGE > 2) {
    // Deep pipeline: before tile kt's last k step every wave waits for tile
    // kt+1 only (tiles kt+2 .. kt+NSTAGE-1 stay in flight: L loads each per
    // wave), and after the barrier refills the stage tile kt has freed with
    // tile kt+NSTAGE (past K: zeros, no memory access).
    constexpr int L = DmaLoader<BM, AL, NW, BK>::PER + NB * DmaLoader<BN, BL, NW, BK>::PER;
    if (nk > 0) {
#pragma unroll
      for (int t = 0; t < NSTAGE; ++t) issue(t);
      wait_vmcnt<(NSTAGE - 1) * L>();
      __builtin_amdgcn_s_waitcnt(0xC07F);
      barrier();
      load_frags(F[0], 0, 0);
    }
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          load_frags(F[(kk + 1) & 1], kt, kk + 1);
        } else if (kt + 1 < nk) {
          wait_vmcnt<(NSTAGE - 2) * L>();
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of tile kt are done
          barrier();
          issue(kt + NSTAGE);
          load_frags(F[0], kt + 1, 0);
        }
        mfmas(F[kk & 1]);
        interleave();
      }
    }
  } else {
    if constexpr (AL == KMAJOR && (BL == KMAJOR || NB == 1)) {
      if (half == 0)
        kloop(std::integral_constant<int, 0>{});
      else
        kloop(std::integral_constant<int, 1>{});
    } else {
      kloop(std::integral_constant<int, 2>{});  // one copy, the half chosen at run time
    }
    if (nk > 0) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) load_frags(F[(kk + 1) & 1], nk - 1, kk + 1);
        mfmas(F[kk & 1]);
        interleave();
      }
    }
  }

  // Epilogue, one 32-row block of the wave's sub-tile at a time, through LDS
  // (idle once every wave is past the K loop): the wave writes its
  // accumulators to its own padded region, where lane l holds row l % 32 and
  // columns 8*q4 + 4*(l / 32) + e of each 32-column tile, and reads them back
  // so that WN/4 consecutive lanes cover one row, four columns each.  The
  // epilogue's loads of saved tensors and its stores then move whole
  // contiguous row segments per instruction, and its saved-tensor loads for
  // the block are issued before any of them is consumed.
  constexpr int LPR = WN / 4;           // lanes per staged row
  constexpr int RPP = 64 / LPR;         // rows per pass
  constexpr int PASSES = 32 / RPP;
  constexpr int PITCH = WN * 4 + 16;    // bytes per staged row (16-byte pad: conflict-free writes)
  static_assert(64 % LPR == 0 && 32 % RPP == 0, "staging layout");
  static_assert(NW * NB * 32 * PITCH <= smem_bytes<BM, BN, WGM, WGN, BK, NB>(), "staging space");
  wait_vmcnt<0>();  // no LDS-direct load (the zero refill included) may land in the staging area
  lds::wait_lgkm0();
  barrier();
  const uint32_t stage = (uint32_t)(wave * NB * 32 * PITCH);
  const int srow = lane / LPR, scol = (lane % LPR) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {acc[b][i][j][4 * q4], acc[b][i][j][4 * q4 + 1], acc[b][i][j][4 * q4 + 2],
                           acc[b][i][j][4 * q4 + 3]};
          const uint32_t off = stage + (uint32_t)(b * 32 * PITCH + (lane & 31) * PITCH +
                                                  (j * 32 + q4 * 8 + (lane >> 5) * 4) * 4);
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(const_cast<lds_u8*>(lds) + off) = v;
        }
    typename Epi::Aux aux[PASSES];
    const int mb = m0 + wm * WM + i * 32, n = n0 + wn * WN + scol;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) epi.load(mb + ps * RPP + srow, n, aux[ps]);
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      float v[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t off = stage + (uint32_t)(b * 32 * PITCH + (ps * RPP + srow) * PITCH + scol * 4);
        const f32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lds + off);
        v[b][0] = x[0];
        v[b][1] = x[1];
        v[b][2] = x[2];
        v[b][3] = x[3];
      }
      epi(mb + ps * RPP + srow, n, v, aux[ps]);
    }
  }
}

// Split tail.  When a launch's tile count leaves its last round of 256 CUs
// at most half full, that round costs about as long as a full one.  The
// last `tail` tiles of the dispatch order are then each computed by two
// work-groups over the two halves of K, so the round takes half as long:
// the halves write fp32 partial tiles to `scratch` ([tail][2][NB][BM][BN]),
// and split_tail_finish_kernel adds them (first half + second half) and runs
// the epilogue.  Requires a tile count that is a multiple of 8 (one equal run
// of tiles per XCD) with tail <= 128.
struct SplitTail {
  float* scratch;  // null: no split
  int full;        // work-groups 0 .. full-1 compute whole tiles
  int tail;        // tiles split in two
};

// fp32 partial tile of a split: v for row m, columns n .. n+3 of tile (m0, n0).
template <int BM, int BN, int NB_>
struct EpiPartial {
  static constexpr int NB = NB_;
  struct Aux {};
  float* base;  // this half's [NB][BM][BN] block
  int m0, n0;
  __device__ __forceinline__ void load(int, int, Aux&) const {}
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& = Aux()) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4 x = {v[b][0], v[b][1], v[b][2], v[b][3]};
      __builtin_nontemporal_store(
          x, reinterpret_cast<f32x4*>(base + ((int64_t)b * BM + (m - m0)) * BN + (n - n0)));
    }
  }
};

// Tile coordinates of split slot `slot` (0 .. tail-1), half of XCD run
// position full/8 + slot/8 on XCD slot%8: the tile that work-group
// (position * 8 + XCD) of an unsplit launch computes.
__device__ __forceinline__ void split_tile(const SplitTail& sp, int slot, int tiles_m, int tiles_n, int& tm, int& tn) {
  gemm::tile_coords((sp.full / 8 + slot / 8) * 8 + slot % 8, tiles_m, tiles_n, tm, tn);
}

// SPLIT: the launch may carry a split tail (instantiated only where a caller
// asks for it, so the plain kernel keeps its register budget).
template <int BM, int BN, int WGM, int WGN, int BK, int AL, int BL, class Epi, bool SPLIT = false>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) gemm_dma_kernel(GemmProblem p, Epi epi, SplitTail sp) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[smem_bytes<BM, BN, WGM, WGN, BK, Epi::NB>()];
  const int w = blockIdx.x;
  if (!SPLIT || w < sp.full) {
    gemm_dma_tile<BM, BN, WGM, WGN, BK, AL, BL, Epi>(p, epi, w, smem);
    return;
  }
  // split work-group s = w - full runs on XCD s % 8 and takes half (s/8) % 2
  // of slot (s/8)/2 * 8 + s % 8
  const int s = w - sp.full, x = s & 7, j = s >> 3;
  const int slot = (j >> 1) * 8 + x, part = j & 1;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  split_tile(sp, slot, tiles_m, tiles_n, tm, tn);
  const int nk = (p.K[0] + BK - 1) / BK + (p.nseg > 1 ? (p.K[1] + BK - 1) / BK : 0);
  const int h0 = nk / 2;
  EpiPartial<BM, BN, Epi::NB> ep{sp.scratch + (int64_t)(slot * 2 + part) * Epi::NB * BM * BN, tm * BM, tn * BN};
  gemm_dma_tile<BM, BN, WGM, WGN, BK, AL, BL, EpiPartial<BM, BN, Epi::NB>, true>(
      p, ep, (sp.full / 8 + slot / 8) * 8 + slot % 8, smem, part ? h0 : 0, part ? nk - h0 : h0);
}

// Sum of the two halves of every split tile, in a fixed order, handed to the
// epilogue: one thread per row and four columns.
template <int BM, int BN, class Epi>
__global__ void __launch_bounds__(256) split_tail_finish_kernel(GemmProblem p, Epi epi, SplitTail sp) {
  constexpr int NB = Epi::NB, Q = BN / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)sp.tail * BM * Q) return;
  const int slot = (int)(i / (BM * Q)), r = (int)(i / Q % BM), c = (int)(i % Q) * 4;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  split_tile(sp, slot, tiles_m, tiles_n, tm, tn);
  const int m = tm * BM + r, n = tn * BN + c;
  if (m >= p.M || n >= p.N) return;
  const float* h0 = sp.scratch + (int64_t)slot * 2 * NB * BM * BN;
  const float* h1 = h0 + NB * BM * BN;
  float v[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(h0 + ((int64_t)b * BM + r) * BN + c);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(h1 + ((int64_t)b * BM + r) * BN + c);
    v[b][0] = a[0] + bb[0];
    v[b][1] = a[1] + bb[1];
    v[b][2] = a[2] + bb[2];
    v[b][3] = a[3] + bb[3];
  }
  typename Epi::Aux aux;
  epi.load(m, n, aux);
  epi(m, n, v, aux);
}

// Tile shape and operand layouts of one problem of a paired launch.
template <int BM_, int BN_, int WGM_, int WGN_, int BK_, int AL_, int BL_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_, AL = AL_, BL = BL_;
  static constexpr int THREADS = 64 * WGM_ * WGN_;
};

// Two independent problems in one launch: work-groups 0 .. tiles1-1 take the
// tiles of problem 1, the rest those of problem 2.  When each problem alone
// would leave part of the chip idle in its last round of tiles, the other's
// tiles fill it.
template <class C1, class E1, class C2, class E2>
__global__ void __launch_bounds__(C1::THREADS, 1)
    gemm_dma_pair_kernel(GemmProblem p1, E1 e1, GemmProblem p2, E2 e2, int tiles1) {
  static_assert(C1::THREADS == C2::THREADS, "both problems run on work-groups of one size");
  constexpr int S1 = smem_bytes<C1::BM, C1::BN, C1::WGM, C1::WGN, C1::BK, E1::NB>();
  constexpr int S2 = smem_bytes<C2::BM, C2::BN, C2::WGM, C2::WGN, C2::BK, E2::NB>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S1 > S2 ? S1 : S2];
  const int w = blockIdx.x;
  if (w < tiles1)
    gemm_dma_tile<C1::BM, C1::BN, C1::WGM, C1::WGN, C1::BK, C1::AL, C1::BL, E1>(p1, e1, w, smem);
  else
    gemm_dma_tile<C2::BM, C2::BN, C2::WGM, C2::WGN, C2::BK, C2::AL, C2::BL, E2>(p2, e2, w - tiles1, smem);
}

// A paired launch whose problem 2 runs its last tile rows as half-width
// tiles: work-groups 0 .. tiles1-1 take problem 1, the next ones problem 2's
// tile rows 0 .. rows2-1 at full width, the rest its remaining rows as
// BM x BN/2 tiles, dispatched last.  When the launch's last round of full
// tiles would leave CUs idle, those rows fill it with twice as many tiles of
// half the work.  Each output element sums the same K tiles in the same
// order as with full-width tiles, so the result is bit-identical.
template <class C1, class E1, class C2, class E2>
__global__ void __launch_bounds__(C1::THREADS, 1)
    gemm_dma_pair_tail_kernel(GemmProblem p1, E1 e1, GemmProblem p2, E2 e2, int tiles1, int rows2) {
  static_assert(C1::THREADS == C2::THREADS, "both problems run on work-groups of one size");
  constexpr int HBN = C2::BN / 2;
  constexpr int S1 = smem_bytes<C1::BM, C1::BN, C1::WGM, C1::WGN, C1::BK, E1::NB>();
  constexpr int S2 = smem_bytes<C2::BM, C2::BN, C2::WGM, C2::WGN, C2::BK, E2::NB>();
  constexpr int S12 = S1 > S2 ? S1 : S2;
  constexpr int S3 = smem_bytes<C2::BM, HBN, C2::WGM, C2::WGN, C2::BK, E2::NB>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S12 > S3 ? S12 : S3];
  const int w = blockIdx.x;
  const int tiles2 = rows2 * ((p2.N + C2::BN - 1) / C2::BN);
  if (w < tiles1) {
    gemm_dma_tile<C1::BM, C1::BN, C1::WGM, C1::WGN, C1::BK, C1::AL, C1::BL, E1>(p1, e1, w, smem);
  } else if (w < tiles1 + tiles2) {
    gemm_dma_tile<C2::BM, C2::BN, C2::WGM, C2::WGN, C2::BK, C2::AL, C2::BL, E2>(p2, e2, w - tiles1, smem, 0, 0, 0,
                                                                              rows2);
  } else {
    const int rows3 = (p2.M + C2::BM - 1) / C2::BM - rows2;
    gemm_dma_tile<C2::BM, HBN, C2::WGM, C2::WGN, C2::BK, C2::AL, C2::BL, E2>(p2, e2, w - tiles1 - tiles2, smem, 0, 0,
                                                                           rows2, rows3);
  }
}

}  // namespace gemm3

// Host-side launcher: grid of ceil(M/BM) * ceil(N/BN) work-groups of 64 * WGM * WGN threads.
template <int BM, int BN, int WGM, int WGN, int BK, int AL, int BL, class Epi>
hipError_t launch_gemm_dma(const GemmProblem& p, const Epi& epi, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  tp_launch((gemm3::gemm_dma_kernel<BM, BN, WGM, WGN, BK, AL, BL, Epi>), dim3(tiles),
            dim3(64 * WGM * WGN), 0, stream, p, epi, gemm3::SplitTail{nullptr, tiles, 0});
  return hipGetLastError();
}

// Scratch floats a split-tail launch of this tile shape needs, or 0 when the
// split does not apply (tile count not a multiple of 8, last round more than
// half full or already full, fewer than two K tiles per half).
template <int BM, int BN, int BK, int NB>
int64_t split_tail_floats(const GemmProblem& p) {
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const int64_t tail = tiles % 256;
  const int nk = (p.K[0] + BK - 1) / BK + (p.nseg > 1 ? (p.K[1] + BK - 1) / BK : 0);
  if (tiles < 256 || tiles % 8 || tail == 0 || tail > 128 || nk < 4) return 0;
  return tail * 2 * NB * BM * BN;
}

// Split-tail launch: the GEMM (whole tiles, then the split halves of the
// last `tail` tiles) and the kernel that finishes those tiles.
template <int BM, int BN, int WGM, int WGN, int BK, int AL, int BL, class Epi>
hipError_t launch_gemm_dma_split(const GemmProblem& p, const Epi& epi, float* scratch, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const int tail = tiles % 256;
  const gemm3::SplitTail sp{scratch, tiles - tail, tail};
  tp_launch((gemm3::gemm_dma_kernel<BM, BN, WGM, WGN, BK, AL, BL, Epi, true>), dim3(tiles + tail),
            dim3(64 * WGM * WGN), 0, stream, p, epi, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)tail * BM * (BN / 4);
  tp_launch((gemm3::split_tail_finish_kernel<BM, BN, Epi>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
            stream, p, epi, sp);
  return hipGetLastError();
}

// Paired launcher: problem 1's tiles (dispatched first) then problem 2's.
template <class C1, class C2, class E1, class E2>
hipError_t launch_gemm_dma_pair(const GemmProblem& p1, const E1& e1, const GemmProblem& p2, const E2& e2,
                                hipStream_t stream) {
  const int t1 = ((p1.M + C1::BM - 1) / C1::BM) * ((p1.N + C1::BN - 1) / C1::BN);
  const int t2 = ((p2.M + C2::BM - 1) / C2::BM) * ((p2.N + C2::BN - 1) / C2::BN);
  if (t1 + t2 == 0) return hipSuccess;
  tp_launch((gemm3::gemm_dma_pair_kernel<C1, E1, C2, E2>), dim3(t1 + t2), dim3(C1::THREADS), 0, stream,
            p1, e1, p2, e2, t1);
  return hipGetLastError();
}

// Tile rows of problem 2 that a paired launch keeps at full width, or -1 when
// the half-width tail does not apply: the launch has more than one round of
// tiles, its last round is more than a quarter and at most half full, and the
// fewest whole tile rows of problem 2 that cover that round's tiles leave at
// least one row whole.  (Measured on gfx950: a half-full last round gains,
// one of 48 tiles loses a little, since so few tiles already run on a chip
// clocked near its maximum.)
template <class C1, class C2>
int pair_tail_rows(const GemmProblem& p1, const GemmProblem& p2) {
  const int t1 = ((p1.M + C1::BM - 1) / C1::BM) * ((p1.N + C1::BN - 1) / C1::BN);
  const int rows = (p2.M + C2::BM - 1) / C2::BM, cols = (p2.N + C2::BN - 1) / C2::BN;
  const int total = t1 + rows * cols, tail = total % 256;
  if (total <= 256 || tail <= 64 || tail > 128 || cols == 0) return -1;
  const int split = (tail + cols - 1) / cols;
  return split < rows ? rows - split : -1;
}

// Paired launcher with problem 2's last tile rows at half width (rows2 from
// pair_tail_rows, at least 0).
template <class C1, class C2, class E1, class E2>
hipError_t launch_gemm_dma_pair_tail(const GemmProblem& p1, const E1& e1, const GemmProblem& p2, const E2& e2,
                                     int rows2, hipStream_t stream) {
  const int t1 = ((p1.M + C1::BM - 1) / C1::BM) * ((p1.N + C1::BN - 1) / C1::BN);
  const int rows = (p2.M + C2::BM - 1) / C2::BM;
  const int t2 = rows2 * ((p2.N + C2::BN - 1) / C2::BN);
  const int t3 = (rows - rows2) * ((p2.N + C2::BN / 2 - 1) / (C2::BN / 2));
  tp_launch((gemm3::gemm_dma_pair_tail_kernel<C1, E1, C2, E2>), dim3(t1 + t2 + t3), dim3(C1::THREADS), 0,
            stream, p1, e1, p2, e2, t1, rows2);
  return hipGetLastError();
}

}  // namespace tp
