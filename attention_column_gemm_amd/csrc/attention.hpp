// Causal grouped-query attention forward of one TP rank's local heads, on the
// gfx950 matrix cores, flash style.
//
// What it computes ([L11] section 4 -- the grasp.study lesson
// "张量并行线性层分片与前反向通信量计算"; [HJ] hjcheng0602.cn "tensorparallel/tp",
// Attention): per sequence and local query head j, with KV head j / (q/kv),
// O = softmax(Q K^T / sqrt(d) + causal mask) V.  Softmax is per head and per
// row, so a rank that holds whole heads needs nothing from other ranks.
//
// How (the row-by-row, O(S)-memory scheme that [LP] "ラブパラ" I.O sketches for
// FlashAttention, laid out for 64-wide waves):
//  * A work-group is 4 waves.  Each wave owns 32 query rows of one head; the
//    waves of a work-group share one KV head (HG query heads of the same
//    group x 4/HG row blocks), so each K/V block is staged in LDS once for all
//    of them.
//  * Keys advance in blocks of 64, loaded straight from HBM into row-major,
//    chunk-swizzled LDS tiles with LDS-direct loads (double buffered; the
//    waves split each block's loads).
//  * S^T = K Q^T is formed with v_mfma_f32_32x32x16_bf16 taking the K
//    fragment as first operand, which leaves one query row per lane (its 64
//    keys split between lanes l and l + 32): row maxima need one cross-half
//    exchange, and the running sums stay per lane until the end.
//  * O^T = V^T P^T uses the probabilities straight from the S registers as the
//    second operand, in the permuted key order those registers hold; the
//    matching V^T operand is read from the row-major V tile with
//    ds_read_b64_tr_b16 in that same order, so P never goes through LDS and V
//    is never stored transposed.
//  * Online softmax in base 2 (scores pre-multiplied by log2(e)/sqrt(d)),
//    exponentials on v_exp_f32 directly; the running output is rescaled only
//    when some row's maximum moved, and blocks wholly inside the causal
//    triangle skip the mask.
//  * Work-groups are ranked by work (later query rows see more keys); the
//    first half of the dispatch order runs heaviest-first and the second half
//    lightest-first, so each CU's two work-groups add up to about the same
//    work.
#pragma once

#include <type_traits>

#include "attn_tiles.hpp"
#include "common.hpp"
#include "lds_dma.hpp"

namespace tp {
namespace attn {

constexpr int BKV = 64;
constexpr int NTHREADS = 256;
// Largest growth (log2 units) of a row's scores over its softmax reference
// before the paired kernel moves the reference and rescales the output.
constexpr float kLazy = 8.0f;

struct AttnArgs {
  const uint16_t* qkv;   // [T, (q + 2kv) d]
  uint16_t* o;           // [T, q d]
  float* lse;            // [b, q, s] or null
  int64_t ld_qkv, ld_o;
  int b, s, q, kv, hg;   // hg: query heads per work-group
  int causal;
  float scale_log2;      // log2(e) / sqrt(d)
  // Load balance when the launch leaves work-group slots empty: the heavier
  // `split` query blocks of every head group are each taken by two
  // work-groups over the two halves of their key blocks; each half leaves
  // its unnormalized output, running maximum and row sums in `part`
  // ([split ny][2][4 waves][D/32 * 16 + 2][64]) and attn_fwd_merge_kernel
  // combines them.
  float* part;
  int split;
  int paired;  // run attn_fwd_paired_kernel (causal, one full round of paired query blocks)
};

// Job J of a split launch (npb query blocks x ny head groups, S of the blocks
// split), heaviest first: for i < S, both halves of block npb-1-i for every
// head group, then whole block npb-1-S-i; the remaining whole blocks follow
// in decreasing order.  part: -1 whole, else the half; slot: i ny + y.
__device__ __forceinline__ void split_job(int J, int npb, int ny, int S, int& pb, int& y, int& part, int& slot) {
  if (J < 3 * ny * S) {
    const int i = J / (3 * ny), r = J % (3 * ny);
    if (r < 2 * ny) {
      pb = npb - 1 - i; part = r / ny; y = r % ny; slot = i * ny + y;
    } else {
      pb = npb - 1 - S - i; part = -1; y = r - 2 * ny; slot = -1;
    }
  } else {
    const int r = J - 3 * ny * S;
    pb = npb - 1 - 2 * S - r / ny; part = -1; y = r % ny; slot = -1;
  }
}

template <int D>
__global__ void __launch_bounds__(NTHREADS, 2) attn_fwd_kernel(AttnArgs a) {
  constexpr int DT = D / 32;                 // 32-wide d tiles of O
  constexpr int KK = D / 16;                 // k steps of S = Q K^T
  constexpr int TILE = BKV * D * 2;          // one K or V block in LDS
  constexpr int STAGE = 2 * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const lds::lds_u8* lds = (const lds::lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int lane = threadIdx.x & 63, hgrp = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv;
  const int sub_per_kv = group / a.hg;
  const int ny = a.b * a.kv * sub_per_kv;
  int pb, y, part = -1, slot = -1;
  if (a.split > 0)
    split_job((int)blockIdx.x, npb, ny, a.split, pb, y, part, slot);
  else
    attnt::causal_block_order(npb, ny, pb, y);
  const int beta = y / (a.kv * sub_per_kv);
  const int rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * a.hg + (wave % a.hg);
  const int pos0 = pb * rows_per_wg;
  const int rp0 = pos0 + (wave / a.hg) * 32;
  const int my_row = rp0 + l32;
  const int64_t tok0 = (int64_t)beta * a.s;
  const uint32_t ldb = (uint32_t)a.ld_qkv * 2u;

  // Q fragments of this lane's row (zero beyond the sequence).
  bf16x8 qf[KK];
  {
    const rsrc_t seq = make_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldb);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint32_t off = (uint32_t)my_row * ldb + (uint32_t)(j * D + kk * 16 + hgrp * 8) * 2u;
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(seq, my_row < a.s ? off : kOOB));
    }
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): keep these out of the block pipeline's counts

  const int kv_end = a.causal ? min(a.s, pos0 + rows_per_wg) : a.s;
  const int nkb_all = (kv_end + BKV - 1) / BKV;
  // a half takes key blocks [kb0, kb0 + nkb)
  const int kb0 = part == 1 ? nkb_all / 2 : 0;
  const int nkb = part < 0 ? nkb_all : (part == 0 ? nkb_all / 2 : nkb_all - nkb_all / 2);
  const u32x4 rkv = lds::sgpr_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldb);
  const uint32_t kcol = (uint32_t)(a.q + g) * D * 2u, vcol = (uint32_t)(a.q + a.kv + g) * D * 2u;
  auto issue = [&](int kb, int st) {
    const uint32_t dst = lds_base + (uint32_t)st * STAGE;
    attnt::dma_tile<D, BKV>(rkv, ldb, (kb0 + kb) * BKV, a.s, kcol, dst, wave, 4);
    attnt::dma_tile<D, BKV>(rkv, ldb, (kb0 + kb) * BKV, a.s, vcol, dst + TILE, wave, 4);
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (nkb > 0) issue(0, 0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    lds::wait_vmcnt<0>();
    lds::wait_lgkm0();
    lds::barrier();  // block kb is in LDS for every wave; every wave is done with block kb-1
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    const int key0 = (kb0 + kb) * BKV;
    if (a.causal && key0 > rp0 + 31) continue;
    const lds::lds_u8* tk = lds + st * STAGE;
    const lds::lds_u8* tv = tk + TILE;
    // S^T for two 32-key tiles
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(attnt::row_frag<D>(tk, 32 * kt, kk), qf[kk], sacc[kt],
                                                           0, 0, 0);
    }
    // scale, mask (only blocks that reach past the diagonal or the sequence), block max
    const bool need_mask = (a.causal && key0 + BKV - 1 > rp0) || key0 + BKV > a.s;
    float bmax = -INFINITY;
    auto scale_max = [&](auto masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kt][r] * a.scale_log2;
          if constexpr (decltype(masked)::value) {
            const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hgrp + (r & 3);
            if (key >= a.s || (a.causal && key > my_row)) x = -INFINITY;
          }
          sacc[kt][r] = x;
          bmax = fmaxf(bmax, x);
        }
    };
    if (need_mask)
      scale_max(std::true_type{});
    else
      scale_max(std::false_type{});
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(sacc[kt][r] - m_use);
        psum += p[r];
      }
      pf[kt][0] = attnt::pack8(p);
      pf[kt][1] = attnt::pack8(p + 8);
    }
    l_run = l_run * alpha + psum;
    // rescale only when some row's maximum moved (alpha == 1 exactly otherwise)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int t = 0; t < DT; ++t)
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(attnt::tr_frag<D>(tv, 32 * kt, t, jj), pf[kt][jj],
                                                            oacc[t], 0, 0, 0);
  }

  if (part >= 0) {  // a half: unnormalized output, running maximum and row sum, [i][lane] order
    float* dst = a.part + ((int64_t)(slot * 2 + part) * 4 + wave) * ((DT * 16 + 2) * 64) + lane;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(t * 16 + e) * 64] = oacc[t][e];
    dst[(DT * 16) * 64] = m_run;
    dst[(DT * 16 + 1) * 64] = l_run;
    return;
  }
  // finalize
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_row < a.s) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = a.o + (tok0 + my_row) * a.ld_o + (int64_t)j * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float v[4] = {oacc[t][4 * q4] * inv, oacc[t][4 * q4 + 1] * inv, oacc[t][4 * q4 + 2] * inv,
                            oacc[t][4 * q4 + 3] * inv};
        Elem<uint16_t>::store4(orow + t * 32 + 8 * q4 + 4 * hgrp, v);
      }
    if (a.lse && hgrp == 0)
      a.lse[((int64_t)beta * a.q + j) * a.s + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

// Merge of the two halves of every split query block, one thread per (slot,
// wave, 32-wide d tile, lane): both halves' values loaded first, each half
// rescaled to the common maximum (exp2, the scores being in log2 units) and
// the halves added in a fixed order (first + second), then normalized and
// stored with the row and head mapping of attn_fwd_kernel.
template <int D>
__global__ void __launch_bounds__(NTHREADS) attn_fwd_merge_kernel(AttnArgs a) {
  constexpr int DT = D / 32, W = (DT * 16 + 2) * 64;
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv, sub_per_kv = group / a.hg;
  const int ny = a.b * a.kv * sub_per_kv;
  const int64_t t = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  if (t >= (int64_t)a.split * ny * 4 * DT * 64) return;
  const int lane = (int)(t & 63), tt = (int)((t >> 6) % DT);
  const int64_t sw = (t >> 6) / DT;
  const int wave = (int)(sw & 3), slot = (int)(sw >> 2);
  const int i = slot / ny, y = slot % ny;
  const int pb = npb - 1 - i;
  const int beta = y / (a.kv * sub_per_kv), rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * a.hg + (wave % a.hg);
  const int my_row = pb * rows_per_wg + (wave / a.hg) * 32 + (lane & 31), hgrp = lane >> 5;
  if (my_row >= a.s) return;
  const float* h0 = a.part + ((int64_t)(slot * 2) * 4 + wave) * W;
  const float* h1 = h0 + 4 * W;
  float x0[16], x1[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    x0[e] = h0[(tt * 16 + e) * 64 + lane];
    x1[e] = h1[(tt * 16 + e) * 64 + lane];
  }
  const float m0 = h0[DT * 16 * 64 + lane], m1 = h1[DT * 16 * 64 + lane];
  const float l0 = h0[(DT * 16 + 1) * 64 + lane] + h0[(DT * 16 + 1) * 64 + (lane ^ 32)];
  const float l1 = h1[(DT * 16 + 1) * 64 + lane] + h1[(DT * 16 + 1) * 64 + (lane ^ 32)];
  const float m = fmaxf(m0, m1);
  const float c0 = m0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - m);
  const float c1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
  const float l = l0 * c0 + l1 * c1;
  const float inv = 1.0f / l;
  uint16_t* orow = a.o + ((int64_t)beta * a.s + my_row) * a.ld_o + (int64_t)j * D + tt * 32;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (x0[4 * q4 + e] * c0 + x1[4 * q4 + e] * c1) * inv;
    Elem<uint16_t>::store4(orow + 8 * q4 + 4 * hgrp, v);
  }
  if (a.lse && hgrp == 0 && tt == 0)
    a.lse[((int64_t)beta * a.q + j) * a.s + my_row] = (m + __log2f(l)) * 0.69314718055994531f;
}

// Causal forward with every work-group given the same work: work-group y of
// job pair pr takes query block pr and then query block npb-1-pr of head
// group y (npb-1-pr is skipped when it is pr), together npb+1 row blocks of
// causal key range, so a single round of work-groups finishes together.  Its
// eight waves are two sets of four: set `par` (0 or 1) runs attn_fwd_kernel's
// four row/head roles on the 64-key blocks 2 i + par of each 128-key
// superblock i, both sets sharing one superblock in LDS ([K even, K odd,
// V even, V odd]).  Wave w of set 0 and wave w of set 1 share a SIMD, and
// set 1 runs half a step behind: in step i set 0 computes the scores of
// its block of superblock i, their softmax and the output product, while
// set 1 first finishes superblock i-1 (softmax and output product of the
// scores it kept) and then computes the scores of superblock i.  Each
// set's matrix instructions thus meet the other set's softmax arithmetic on
// the SIMD instead of its own.  V odd is read one step later than the
// rest of a superblock, so it is loaded one step later too.  At the end of
// a query block set 1 finishes its last block, then hands its unnormalized
// output, running maximum and row sums to set 0 through LDS, which merges
// them (each half rescaled to the common maximum, first + second),
// normalizes and stores.
template <int D>
__global__ void __launch_bounds__(2 * NTHREADS, 1) attn_fwd_paired_kernel(AttnArgs a) {
  constexpr int DT = D / 32;                 // 32-wide d tiles of O
  constexpr int KK = D / 16;                 // k steps of S = Q K^T
  constexpr int TILE = BKV * D * 2;          // one 64-key K or V block in LDS
  constexpr int STAGE = 4 * TILE;            // one 128-key superblock
  constexpr int QT = 32 * D * 2;              // one wave's [32][D] Q tile
  constexpr int HT = DT / 2;                  // d tiles of 32 that each set merges
  constexpr int HALF = HT * 16 * 64 * 4;      // bytes of a wave's unnormalized output on those tiles
  constexpr int HROW = D + 16;                // padded half row (D / 2 bf16) of the staged output
  static_assert(4 * 2 * HALF <= STAGE, "both sets' handovers fit in one stage");
  static_assert(32 * HROW <= HALF, "a staged half row block fits in a handover");
  static_assert(4 * 256 * 4 <= TILE, "both sets' maxima and sums fit in one tile");
  // two superblock stages, then the four row/head roles' Q tiles
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + 4 * QT];
  const lds::lds_u8* lds = (const lds::lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int lane = threadIdx.x & 63, hgrp = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int par = wave >> 2, w4 = wave & 3;
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv;
  const int sub_per_kv = group / a.hg;
  const int ny = a.b * a.kv * sub_per_kv;
  const int y = (int)blockIdx.x % ny, pr = (int)blockIdx.x / ny;
  const int beta = y / (a.kv * sub_per_kv);
  const int rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * a.hg + (w4 % a.hg);
  const int64_t tok0 = (int64_t)beta * a.s;
  const uint32_t ldb = (uint32_t)a.ld_qkv * 2u;
  const rsrc_t seq = make_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldb);
  const u32x4 rkv = lds::sgpr_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldb);
  const uint32_t kcol = (uint32_t)(a.q + g) * D * 2u, vcol = (uint32_t)(a.q + a.kv + g) * D * 2u;

  // the job's query blocks and their 128-key superblocks
  const int pbA = pr, pbB = npb - 1 - pr;
  auto nkb_of = [&](int pb) { return (min(a.s, (pb + 1) * rows_per_wg) + BKV - 1) / BKV; };
  const int nsbA = (nkb_of(pbA) + 1) / 2;
  const int nsbB = pbB != pbA ? (nkb_of(pbB) + 1) / 2 : 0;
  const int total = nsbA + nsbB;
  // Loads of a superblock's four 64-key tiles [K even, K odd, V even,
  // V odd], TILE / 1024 one-KiB instructions each, dealt out over the eight
  // wave slots; slot w's share of a tile is PER_TILE instructions, part u
  // being instruction w + 8 (u % PER_TILE) of tile u / PER_TILE.
  static_assert(TILE % 8192 == 0, "each tile splits evenly over the eight waves");
  constexpr int PER_TILE = TILE / 1024 / 8;
  // every instruction i = w + 8 p this wave issues has i = wave mod 4
  const uint32_t kv_lane = attnt::dma_lane_off<D>(ldb, wave);
  auto issue_part = [&](int idx, int st, int u, int w) {
    const int sb = idx < nsbA ? idx : idx - nsbA;
    const int tile = u / PER_TILE, i = w + 8 * (u % PER_TILE);
    const int row0 = sb * 2 * BKV + (tile & 1) * BKV;
    attnt::dma_tile_part_at<D>(rkv, ldb, row0, tile < 2 ? kcol : vcol,
                               lds_base + (uint32_t)st * STAGE + (uint32_t)tile * TILE, i, kv_lane);
  };
  // Step idx's loads: K even, K odd and V even of superblock idx + 1 into
  // the other stage (read last in step idx - 1), and V odd of superblock
  // idx into this stage (its previous V odd was read by set 1 in step
  // idx - 1); both are waited for at the top of step idx + 1.  Set 0
  // finishes its step's work earlier than set 1, which carries the softmax
  // of its previous block, so each set 0 wave also issues its set 1
  // partner's share of superblock idx + 1: a wave issuing LDS-direct loads
  // is held until the CU's L2-to-LDS path accepts them, and set 0 would
  // otherwise spend that time at the barrier.
  auto issue = [&](int idx, int st, bool next) {
    if (next) {
#pragma unroll
      for (int u = 0; u < 3 * PER_TILE; ++u) {
        if (par == 0) {
          issue_part(idx + 1, st ^ 1, u, wave);
          issue_part(idx + 1, st ^ 1, u, wave + 4);
        }
      }
    }
#pragma unroll
    for (int u = 3 * PER_TILE; u < 4 * PER_TILE; ++u) issue_part(idx, st, u, wave);
  };
  // Q of query block pb: role w4's tile (rows rp0 .. rp0 + 31 of head j,
  // zeros beyond the sequence) in Q slot w4, half of its D / 16 one-KiB
  // instructions from each set.
  auto issue_q = [&](int pb) {
    const int rq0 = pb * rows_per_wg + (w4 / a.hg) * 32;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
      attnt::dma_tile_part<D>(rkv, ldb, rq0, a.s, (uint32_t)j * D * 2u, lds_base + 2 * STAGE + (uint32_t)w4 * QT,
                              par * (D / 32) + u);
  };
  const lds::lds_u8* tq = lds + 2 * STAGE + w4 * QT;

  // Each set runs its own copy of the loop (the same barriers in the same
  // order), so neither copy's registers are shaped by the other's.
  auto run = [&](auto set) {
    constexpr int P = decltype(set)::value;
    bf16x8 qf[KK];       // this role's Q fragments, read from its LDS tile once per query block
    f32x16 oacc[DT];
    f32x16 sacc[2];      // the scores of this wave's current block (set 1: kept to the next step)
    float m_run = -INFINITY, l_run = 0.0f;
    int rp0 = 0, my_row = 0, nkb = 0, key0p = 0;
    bool pend = false;   // set 1: sacc holds the scores of block key0p, not yet taken further
    auto scores = [&](const lds::lds_u8* tk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(attnt::row_frag<D>(tk, 32 * kt, kk),
                                                             qf[kk], sacc[kt], 0, 0, 0);
    };
    // Online softmax in base 2 against a per-row reference m_run that only
    // moves when the block's scaled maximum exceeds it by more than kLazy:
    // probabilities stay below 2^kLazy, and the running output is rescaled
    // only on such moves.  The score scale rides on the exponent's FMA, and
    // the block maximum is taken on the raw scores.  Then O += P V.
    auto softmax_pv = [&](int key0, const lds::lds_u8* tv) {
      const bool need_mask = key0 + BKV - 1 > rp0 || key0 + BKV > a.s;
      float bmax = -INFINITY;
      auto raw_max = [&](auto masked) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (decltype(masked)::value) {
              const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hgrp + (r & 3);
              if (key >= a.s || key > my_row) sacc[kt][r] = -INFINITY;
            }
            bmax = fmaxf(bmax, sacc[kt][r]);
          }
      };
      if (need_mask)
        raw_max(std::true_type{});
      else
        raw_max(std::false_type{});
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32)) * a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(bmax > m_run + kLazy)) {
        const float m_new = bmax > m_run + kLazy ? bmax : m_run;
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.0f : m_run;
      float psum = 0.0f;
      bf16x8 pf[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], a.scale_log2, -m_use));
          psum += p[r];
        }
        pf[kt][0] = attnt::pack8(p);
        pf[kt][1] = attnt::pack8(p + 8);
      }
      l_run += psum;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int t = 0; t < DT; ++t)
            oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(attnt::tr_frag<D>(tv, 32 * kt, t, jj), pf[kt][jj],
                                                              oacc[t], 0, 0, 0);
    };
    if (total > 0) {
      issue_q(pbA);
#pragma unroll
      for (int u = 0; u < 3 * PER_TILE; ++u) issue_part(0, 0, u, wave);
    }
    for (int idx = 0; idx < total; ++idx) {
      const int st = idx & 1;
      const bool inB = idx >= nsbA;
      const int sb = inB ? idx - nsbA : idx;
      const int pb = inB ? pbB : pbA;
      lds::wait_vmcnt<0>();
      lds::wait_lgkm0();
      lds::barrier();  // this step's tiles are in LDS; every wave is done with the stages they replace
      if (sb == 0) {   // a new query block (its Q tiles are in LDS): fresh state
        rp0 = pb * rows_per_wg + (w4 / a.hg) * 32;
        my_row = rp0 + l32;
        nkb = nkb_of(pb);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = attnt::row_frag<D>(tq, 0, kk);
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
        m_run = -INFINITY;
        l_run = 0.0f;
      }
      const int kb = 2 * sb + par;
      const int key0 = kb * BKV;
      const bool act = kb < nkb && key0 <= rp0 + 31;
      if constexpr (P == 0) {
        if (act) {
          scores(lds + st * STAGE);
          softmax_pv(key0, lds + st * STAGE + 2 * TILE);
        }
      } else {
        if (pend) softmax_pv(key0p, lds + (st ^ 1) * STAGE + 3 * TILE);
        pend = act;
        if (act) {
          scores(lds + st * STAGE + TILE);
          key0p = key0;
        }
      }
      // The loads go out after the matrix instructions: a wave issuing
      // LDS-direct loads is held until the CU's L2-to-LDS path (tens of bytes
      // per clock) accepts them, and held there the MFMAs it has already
      // issued keep the matrix unit busy.
      lds::wait_lgkm0();
      issue(idx, st, idx + 1 < total);
      if (sb + 1 < (inB ? nsbB : nsbA)) continue;
      // The query block is done.  Set 1 takes its last block further (its
      // V odd tile has arrived at the barrier) while the next block's Q tiles
      // load (every score product of this block is done); this stage and the
      // other stage's V odd slot (idle until the next step's loads) are free
      // once every wave has passed the second barrier.
      lds::wait_vmcnt<0>();
      lds::wait_lgkm0();
      lds::barrier();
      if (idx + 1 < total) issue_q(pbB);
      if constexpr (P == 1) {
        if (pend) softmax_pv(key0p, lds + st * STAGE + 3 * TILE);
        pend = false;
      }
      lds::wait_lgkm0();
      lds::barrier();
      // Each set merges and stores half of the d columns, set 0 the first
      // HT tiles of 32 and set 1 the rest, so each hands the other half of
      // its unnormalized output over through this stage's memory (role w4's
      // share: set 1's handover, then set 0's) and its maxima and sums
      // through the other stage's V odd slot.
      uint8_t* const wbuf = smem + st * STAGE + w4 * (2 * HALF);
      float* const give = reinterpret_cast<float*>(wbuf + (P == 0 ? HALF : 0)) + lane;
      uint8_t* const tbuf = wbuf + (P == 0 ? 0 : HALF);
      float* const take = reinterpret_cast<float*>(tbuf) + lane;
      float* const ml = reinterpret_cast<float*>(smem + (st ^ 1) * STAGE + 3 * TILE) + w4 * 256 + lane;
      constexpr int tg = P == 0 ? HT : 0, tm = P == 0 ? 0 : HT;  // first tile given, first tile merged
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) give[(t * 16 + e) * 64] = oacc[tg + t][e];
      ml[P * 128] = m_run;
      ml[P * 128 + 64] = l_run;
      lds::wait_lgkm0();
      lds::barrier();
      {
        const float mo = ml[(1 - P) * 128], lo = ml[(1 - P) * 128 + 64];
        const float m = fmaxf(m_run, mo);
        const float c0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
        const float c1 = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - m);
        const float l = l_run * c0 + lo * c1;
        const float l_tot = l + __shfl_xor(l, 32);
        const float inv = 1.0f / l_tot;
        // The other set's half into registers, then the merged, normalized
        // bf16 half rows into the same memory ([32][D / 2] with padded
        // rows), read back so that each store covers whole half rows.
        float x1[HT][16];
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) x1[t][e] = take[(t * 16 + e) * 64];
        lds::wait_lgkm0();
        asm volatile("" ::: "memory");  // every lane's reads before any lane's writes
        lds::lds_u8* const wl = (lds::lds_u8*)tbuf;
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (oacc[tm + t][4 * q4 + e] * c0 + x1[t][4 * q4 + e] * c1) * inv;
            u32x2 w;
            w[0] = pack_bf16x2(v[0], v[1]);
            w[1] = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(wl + l32 * HROW +
                                                                        (t * 32 + 8 * q4 + 4 * hgrp) * 2) = w;
          }
        lds::wait_lgkm0();
        asm volatile("" ::: "memory");
        constexpr int CPR = D / 16, RPI = 64 / CPR;  // 16-byte chunks per half row, half rows per pass
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int r = it * RPI + lane / CPR, c = lane % CPR;
          const u32x4 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(wl + r * HROW + c * 16);
          if (rp0 + r < a.s)
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(a.o + (tok0 + rp0 + r) * a.ld_o + (int64_t)j * D +
                                                                  tm * 32 + c * 8));
        }
        if (P == 0 && a.lse && hgrp == 0 && my_row < a.s)
          a.lse[((int64_t)beta * a.q + j) * a.s + my_row] = (m + __log2f(l_tot)) * 0.69314718055994531f;
      }
    }
  };
  if (par == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
}

}  // namespace attn

// Whether the causal forward runs as attn_fwd_paired_kernel: one round of
// equal work-groups (pairs of query blocks) fills every CU.
inline bool attn_fwd_paired(int s, int causal, int b, int q, int kv, int hg) {
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (s + rows_per_wg - 1) / rows_per_wg;
  const int64_t jobs = (int64_t)((npb + 1) / 2) * b * kv * ((q / kv) / hg);
  return causal && npb >= 2 && jobs >= 256;
}

// Query blocks of the forward launch worth splitting (AttnArgs::split): the
// heavier half for a causal mask when the unsplit launch leaves some of its
// 512 work-group slots (two per CU) empty, none otherwise; and the floats of
// AttnArgs::part.
inline int attn_fwd_split(int s, int causal, int b, int q, int kv, int hg) {
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (s + rows_per_wg - 1) / rows_per_wg;
  const int64_t wgs = (int64_t)npb * b * kv * ((q / kv) / hg);
  return causal && wgs < 512 ? npb / 2 : 0;
}
inline int64_t attn_fwd_part_floats(int b, int q, int kv, int hg, int split, int d) {
  return (int64_t)split * b * kv * ((q / kv) / hg) * 2 * 4 * ((d / 32) * 16 + 2) * 64;
}

template <int D>
hipError_t launch_attn_fwd(const attn::AttnArgs& a, hipStream_t stream) {
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int ny = a.b * a.kv * ((a.q / a.kv) / a.hg);
  if (npb == 0 || ny == 0) return hipSuccess;
  if (a.paired) {
    tp_launch((attn::attn_fwd_paired_kernel<D>), dim3(((npb + 1) / 2) * ny), dim3(2 * attn::NTHREADS), 0,
              stream, a);
    return hipGetLastError();
  }
  if (a.split == 0) {
    tp_launch((attn::attn_fwd_kernel<D>), dim3(npb, ny), dim3(attn::NTHREADS), 0, stream, a);
    return hipGetLastError();
  }
  tp_launch((attn::attn_fwd_kernel<D>), dim3((npb + a.split) * ny), dim3(attn::NTHREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)a.split * ny * 4 * (D / 32) * 64;
  tp_launch((attn::attn_fwd_merge_kernel<D>), dim3((unsigned)((n + attn::NTHREADS - 1) / attn::NTHREADS)),
            dim3(attn::NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tp
