// Causal grouped-query attention backward of one TP rank's local heads, on
// the gfx950 matrix cores, flash style.
//
// What it computes ([HJ] hjcheng0602.cn "tensorparallel/tp", Attention,
// single-card backward; [LP] "ラブパラ" I.O on recomputing the scores in the
// backward pass): per sequence and local query head j with KV head
// g = j / (q/kv), scale c = 1/sqrt(d), P = softmax(c Q K^T + causal mask),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta_i = rowsum(dO * O)_i,
//   dQ = c dS K,  dK = c dS^T Q,
// with the KV gradients summed over the query heads of the group.  P is
// recomputed from the forward's per-row log-sum-exp; Delta_i equals
// rowsum(P * dP)_i because O = P V.
//
// Three kernels:
//  * stats: per (sequence, head, row) the pair {lse * log2(e), Delta}.
//  * dK/dV: a work-group owns 32 keys of one KV head, staged once in LDS; its
//    eight waves (two per SIMD) take every eighth (query head, 32-row query
//    tile) item of the causal range, last query tile first, each wave
//    streaming its own Q and dO tiles into LDS with LDS-direct loads, and
//    the eight waves' partial sums are added in a fixed order through LDS at
//    the end (deterministic, no atomics).  The causal key blocks but the
//    lightest eighth (the first ones see the most queries) are split over
//    two work-groups, each taking half of the items, and the jobs go out in
//    decreasing order of work; a small kernel adds the two halves in a fixed
//    order.
//  * dQ: the forward's layout (waves own 32 query rows; the work-group shares
//    64-key K and V blocks in LDS).  Causal, where the tiles fit in memory
//    that the final GEMM writes later, dK/dV hands its dS tiles over instead
//    (transposed on the matrix cores into the register image dQ's products
//    take) and dQ loads them rather than recomputing the scores.
// Operand layouts: with v_mfma_f32_32x32x16_bf16 computing C[i][j] += sum_k
// X[i][k] Y[j][k], lane l holding column j = l % 32 of C, the score tile is
// formed so that the lane's column is the index the next product keeps
// (keys for dK/dV, queries for dQ) and the contracted index lies in its
// registers; those registers are used directly as the Y operand of the
// next product, in a permuted k order, and the matching X operand (Q^T,
// dO^T or K^T) is read with ds_read_b64_tr_b16 from the row-major LDS tile
// in that same order, so no operand tile is ever stored transposed.
#pragma once

#include <type_traits>

#include "attn_tiles.hpp"
#include "common.hpp"
#include "lds_dma.hpp"

namespace tp {
namespace attnb {

using lds::lds_u8;
using lds::v4i16;
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
using attnt::dma4;
using attnt::dma_tile;
using attnt::pack8;
using attnt::row_frag;
using attnt::tile_off;
using attnt::tr_frag;

constexpr int NTHREADS = 256;
constexpr int KEY_BLOCK = 32;   // keys per dK/dV work-group
constexpr int Q_TILE = 32;      // query rows per dK/dV item
constexpr int DQ_KEYS = 64;     // keys per dQ block


struct BwdArgs {
  const uint16_t* qkv;  // [T, (q + 2kv) d] forward projections
  const uint16_t* o;    // [T, q d] forward output
  const uint16_t* dO;   // [T, q d] gradient of O
  const float* lse;     // [b, q, s] forward log-sum-exp (natural log)
  float* stats;         // [b, q, s, 2] {lse * log2(e), Delta}
  uint16_t* dqkv;       // [T, (q + 2kv) d]
  int64_t ld_qkv, ld_o;
  int b, s, q, kv;
  int causal;
  float scale;       // 1 / sqrt(d)
  float scale_log2;  // log2(e) / sqrt(d)
  // dK/dV load balance: key blocks 0 .. split-1 of every (sequence, KV head),
  // the ones that see the most queries, are each taken by two work-groups
  // over the two halves of their items; the halves' fp32 sums go to dkv_part
  // ([b kv split][2][2 D/32][16][64]) and attn_bwd_dkv_combine_kernel adds them.
  float* dkv_part;
  int split;
  // dQ load balance: the heavier dq_split query blocks of every (sequence,
  // head group) are each taken by two work-groups over the two halves of
  // their key blocks; the halves' fp32 sums go to dq_part
  // ([dq_split ny][2][4 waves][D/32 * 16][64]) and attn_bwd_dq_combine_kernel
  // adds them.
  float* dq_part;
  int dq_split;
  // dS tiles handed from dK/dV to dQ (causal only, when they fit): dK/dV
  // stores every item's bf16 dS tile (32 queries x 32 keys, 2 KiB, in the
  // register image dQ's products take: the first 1 KiB holds each lane's
  // first eight values, the second its last eight, 16 bytes per lane), and
  // attn_bwd_dq_ds_kernel loads them straight into registers and computes
  // dQ = c dS K from them.  Tile t of
  // (sequence beta, head j, query tile qt, key block kb <= qt) is
  // (beta q + j) T + qt (qt + 1) / 2 + kb with T = nqt (nqt + 1) / 2 tiles per
  // head; tiles t < ds_t0 sit at ds_a + 2 KiB t, the rest at
  // ds_b + 2 KiB (t - ds_t0).
  uint8_t* ds_a;
  uint8_t* ds_b;
  int64_t ds_t0;
  int ds_path;
};

// 2 KiB dS tile t of the hand-over (see BwdArgs::ds_a).
__device__ __forceinline__ uint8_t* ds_tile(const BwdArgs& a, int64_t t) {
  return t < a.ds_t0 ? a.ds_a + t * 2048 : a.ds_b + (t - a.ds_t0) * 2048;
}

// Job j of the dQ launch (npb query blocks x ny head groups, dq_split of the
// blocks split), heaviest first: for i < dq_split, both halves of block
// npb-1-i for every head group, then whole block npb-1-dq_split-i; the
// remaining whole blocks follow in decreasing order.  part: -1 whole, else
// the half; slot: index of a split block (i ny + y).
__device__ __forceinline__ void dq_job(int J, int npb, int ny, int S, int& pb, int& y, int& part, int& slot) {
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

// ---- stats -------------------------------------------------------------------
// Row r = (beta q + j) s + i: stats[2r] = lse * log2(e), stats[2r+1] = Delta.
// D/8 lanes per row, each with one 16-byte load of dO and of O per row (read
// once: sc1 policy, through descriptors over the whole tensors, which the
// host keeps under 2^31 bytes); a work-group takes STATS_ROWS consecutive
// groups of rows and issues all their loads before using any.  The eight
// products of a lane are added in element order and folded with cross-lane
// adds, and lane 0 of the row stores the pair as one 8-byte store.
constexpr int STATS_ROWS = 4;
template <int D>
__global__ void __launch_bounds__(NTHREADS) attn_bwd_stats_kernel(BwdArgs a, int64_t nrows) {
  constexpr int LPR = D / 8, RPG = NTHREADS / LPR;
  const int sub = threadIdx.x % LPR;
  const uint32_t bytes = (uint32_t)((int64_t)a.b * a.s * a.ld_o * 2);
  const rsrc_t rd = make_rsrc(a.dO, bytes), ro = make_rsrc(a.o, bytes);
  u32x4 x[STATS_ROWS], y[STATS_ROWS];
  float lse[STATS_ROWS];
#pragma unroll
  for (int u = 0; u < STATS_ROWS; ++u) {
    const int64_t r = ((int64_t)blockIdx.x * STATS_ROWS + u) * RPG + threadIdx.x / LPR;
    lse[u] = 0.0f;
    uint32_t off = kOOB;
    if (r < nrows) {
      if (sub == 0) lse[u] = a.lse[r];
      const int64_t i = r % a.s, j = (r / a.s) % a.q, beta = r / ((int64_t)a.s * a.q);
      off = (uint32_t)(((beta * a.s + i) * a.ld_o + j * D + sub * 8) * 2);
    }
    x[u] = __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 2 /* sc1 */);
    y[u] = __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 2 /* sc1 */);
  }
#pragma unroll
  for (int u = 0; u < STATS_ROWS; ++u) {
    const int64_t r = ((int64_t)blockIdx.x * STATS_ROWS + u) * RPG + threadIdx.x / LPR;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += bf16lo(x[u][w]) * bf16lo(y[u][w]);
      acc += bf16hi(x[u][w]) * bf16hi(y[u][w]);
    }
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
    if (r < nrows && sub == 0) {
      const f32x2_t v = {lse[u] * 1.4426950408889634f, acc};
      *reinterpret_cast<f32x2_t*>(a.stats + 2 * r) = v;
    }
  }
}

// ---- dK, dV ----------------------------------------------------------------
// Eight waves (two per SIMD, so one wave's exponentials and loads overlap the
// other's MFMAs) share one 32-key block: its K and V rows sit in LDS once,
// and each wave streams the Q and dO tiles of every eighth item into its own
// LDS slot.
constexpr int DKV_WAVES = 8;
template <int D>
__global__ void __launch_bounds__(64 * DKV_WAVES, 1) attn_bwd_dkv_kernel(BwdArgs a) {
  constexpr int DT = D / 32, KK = D / 16;
  constexpr int TILE = Q_TILE * D * 2;   // one 32-row tile
  constexpr int TI = TILE / 1024;        // its LDS-direct instructions
  constexpr int SLOT = 2 * TILE + 256;   // a wave's Q tile, dO tile, 32 x {lse2, Delta}
  constexpr int KV_BYTES = 2 * TILE;     // the block's K and V rows
  constexpr int LDS_BYTES = KV_BYTES + DKV_WAVES * SLOT;
  constexpr int PART = 2 * DT * 16 * 64 * 4;  // one wave's dK and dV partial sums
  static_assert(4 * PART <= LDS_BYTES, "reduction space");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const lds_u8* lds = (const lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Job J of the 1-D grid, in decreasing order of work: the two halves of a
  // split key block i < split (work (nkb - i) / 2 each) and the whole blocks
  // split .. nkb-1 (work nkb - kb) merged by work, halves first on ties; each
  // entry of that order covers every (sequence, KV head), b kv jobs.
  const int nkb = (a.s + KEY_BLOCK - 1) / KEY_BLOCK;
  const int BG = a.b * a.kv, J = blockIdx.x;
  const int u = J / BG, bg = J % BG;
  int kb = 0, part = -1;  // part: -1 whole, else the half
  {
    int i = 0, w = a.split, pos = 0;  // next split block, next whole block, entries passed
    for (int step = 0; step < nkb; ++step) {  // nkb = split + (nkb - split) entries at most
      const bool take_split = i < a.split && (w >= nkb || (nkb - i) >= 2 * (nkb - w));
      if (take_split) {
        if (u < pos + 2) { kb = i; part = u - pos; break; }
        pos += 2;
        ++i;
      } else {
        if (u == pos) { kb = w; break; }
        pos += 1;
        ++w;
      }
    }
  }
  const int k0 = kb * KEY_BLOCK;
  const int beta = bg / a.kv, g = bg % a.kv;
  const int group = a.q / a.kv;
  const int64_t tok0 = (int64_t)beta * a.s;
  const uint32_t ldq = (uint32_t)a.ld_qkv * 2u, ldo = (uint32_t)a.ld_o * 2u;
  const u32x4 rq = lds::sgpr_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldq);
  const u32x4 rdo = lds::sgpr_rsrc(a.dO + tok0 * a.ld_o, (uint32_t)a.s * ldo);
  const u32x4 rst = lds::sgpr_rsrc(a.stats + (int64_t)beta * a.q * a.s * 2, (uint32_t)a.q * a.s * 8u);

  // the block's K and V rows (zeros past the sequence), loaded once
  dma_tile<D, KEY_BLOCK>(rq, ldq, k0, a.s, (uint32_t)(a.q + g) * D * 2u, lds_base, wave, DKV_WAVES);
  dma_tile<D, KEY_BLOCK>(rq, ldq, k0, a.s, (uint32_t)(a.q + a.kv + g) * D * 2u, lds_base + TILE, wave, DKV_WAVES);
  lds::wait_vmcnt<0>();
  lds::barrier();
  const lds_u8* tkey = lds;
  const lds_u8* tval = lds + TILE;

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[t][e] = dv[t][e] = 0.0f;

  const int nqt = (a.s + Q_TILE - 1) / Q_TILE;
  const int qt0 = a.causal ? (k0 / Q_TILE) : 0;
  const int ntile = nqt - qt0;
  const int nitems = group * ntile;
  const uint32_t slot = lds_base + (uint32_t)(KV_BYTES + wave * SLOT);
  const lds_u8* tq = lds + (KV_BYTES + wave * SLOT);
  const lds_u8* tdo = tq + TILE;
  const lds_u8* tst = tq + 2 * TILE;

  // items run from the last query tile backwards, so the work-groups of one
  // KV head (all key blocks) read the same Q and dO tiles at about the same
  // time and share them in L2; a half takes one half of the items
  const int n_begin = part == 1 ? nitems / 2 : 0, n_end = part == 0 ? nitems / 2 : nitems;
  // item n = (head hq, tile index ti) with n = hq ntile + ti, advanced by
  // DKV_WAVES per pass without a division
  int hq = (n_begin + wave) / ntile, ti = (n_begin + wave) % ntile;
  for (int n = n_begin + wave; n < n_end; n += DKV_WAVES) {
    const int j = g * group + hq;
    const int i0 = (nqt - 1 - ti) * Q_TILE;
    for (ti += DKV_WAVES; ti >= ntile; ti -= ntile) ++hq;
    lds::wait_lgkm0();  // this wave's reads of its slot are done
    // the tiles' TI instructions, their per-lane offsets from the loop
    // invariants of dma_lane_off (rows past the sequence read zeros through
    // the descriptors' bounds): dO and the statistics first, then Q, so that
    // dP's products run while the Q tile is still landing
#pragma unroll
    for (int i = 0; i < TI; ++i)
      attnt::dma_tile_part_at<D>(rdo, ldo, i0, (uint32_t)j * D * 2u, slot + TILE, i, attnt::dma_lane_off<D>(ldo, i));
    {  // lanes 2i, 2i+1: the {lse2, Delta} pair of row i0 + i
      const int row = i0 + (lane >> 1);
      dma4(rst, row < a.s ? ((uint32_t)j * a.s + row) * 8u + (lane & 1) * 4u : kOOB, slot + 2 * TILE);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
      attnt::dma_tile_part_at<D>(rq, ldq, i0, (uint32_t)j * D * 2u, slot, i, attnt::dma_lane_off<D>(ldq, i));

    // dP = dO V^T and S = Q K^T for 32 queries x 32 keys: lane = key, registers = queries
    f32x16 sacc, pacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = pacc[e] = 0.0f;
    lds::wait_vmcnt<TI>();  // dO and the statistics have landed
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(tdo, 0, kk), row_frag<D>(tval, 0, kk), pacc, 0, 0,
                                                     0);
    asm volatile("" : "+v"(pacc));  // dP's products stay ahead of the wait for Q
    lds::wait_vmcnt<0>();   // and Q
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(tq, 0, kk), row_frag<D>(tkey, 0, kk), sacc, 0, 0, 0);
    // P = exp2(S c log2e - lse2), dS = P (dP - Delta); register r holds query 8(r/4) + 4h + r%4.
    // Items wholly inside the sequence and below the causal diagonal skip the mask.
    const int key = k0 + l32;
    const bool full = i0 + Q_TILE <= a.s && (!a.causal || k0 + KEY_BLOCK - 1 <= i0);
    float p[16], ds[16];
    auto probs = [&](auto masked) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ir = 8 * q4 + 4 * h;  // first of this group's four queries within the tile
        const f32x4 s0 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(tst + ir * 8);
        const f32x4 s1 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(tst + ir * 8 + 16);
        const float lse2[4] = {s0.x, s0.z, s1.x, s1.z}, dlt[4] = {s0.y, s0.w, s1.y, s1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e, qi = i0 + ir + e;
          p[r] = __builtin_amdgcn_exp2f(sacc[r] * a.scale_log2 - lse2[e]);
          if constexpr (decltype(masked)::value) {
            if (!(qi < a.s && (!a.causal || key <= qi))) p[r] = 0.0f;
          }
          ds[r] = p[r] * (pacc[r] - dlt[e]);
        }
      }
    };
    if (full)
      probs(std::false_type{});
    else
      probs(std::true_type{});
    bf16x8 pf[2], df[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      pf[jj] = pack8(p + 8 * jj);
      df[jj] = pack8(ds + 8 * jj);
    }
    if (a.ds_path) {
      // The item's dS tile for the dQ kernel, before the products below,
      // whose time covers the stores' write acknowledgement, transposed on
      // the matrix cores: with dS as the first operand (row = key, k = the
      // query order of the registers) and a 0/1 permutation matrix as the
      // second, the product holds dS[query][key] with lane = query and
      // registers = keys in the order dQ's products read K^T, exactly
      // (products with 1 and sums with 0).  Query 16 jj + 8 (m / 4) + 4 h +
      // m % 4 of lane (key, h) sits at k = 8 h + m of df[jj], so operand lane
      // (row, hy) holds 1 at position m when row = 16 jj + 8 (m / 4) + 4 hy +
      // m % 4.
      f32x16 tr;
#pragma unroll
      for (int e = 0; e < 16; ++e) tr[e] = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        u16x8 pm;
#pragma unroll
        for (int m = 0; m < 8; ++m)
          pm[m] = l32 == 16 * jj + 8 * (m >> 2) + 4 * h + (m & 3) ? (uint16_t)0x3F80 : (uint16_t)0;
        tr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df[jj], __builtin_bit_cast(bf16x8, pm), tr, 0, 0, 0);
      }
      const int qt = i0 / Q_TILE;
      uint8_t* dst = ds_tile(a, ((int64_t)beta * a.q + j) * ((int64_t)nqt * (nqt + 1) / 2) + (int64_t)qt * (qt + 1) / 2 +
                                    kb) + lane * 16;
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = tr[e];
        hi[e] = tr[8 + e];
      }
      *reinterpret_cast<bf16x8*>(dst) = pack8(lo);
      *reinterpret_cast<bf16x8*>(dst + 1024) = pack8(hi);
    }
    // dV^T += dO^T P and dK^T += Q^T dS: lane = key, registers = head dims
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tdo, 0, dt, jj), pf[jj], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tq, 0, dt, jj), df[jj], dk[dt], 0, 0, 0);
      }
  }

  // add the eight waves' partial sums in a fixed order, (w0+w4) + (w1+w5) +
  // (w2+w6) + (w3+w7), through LDS in two rounds, and store
  float* red = reinterpret_cast<float*>(smem);  // [4][2 DT][16][64]
  auto slot_of = [&](int w, int u, int e) { return ((w * 2 * DT + u) * 16 + e) * 64 + lane; };
  lds::wait_lgkm0();
  __syncthreads();
  if (wave >= 4) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[slot_of(wave - 4, t, e)] = dk[t][e];
        red[slot_of(wave - 4, DT + t, e)] = dv[t][e];
      }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dk[t][e] += red[slot_of(wave, t, e)];
        dv[t][e] += red[slot_of(wave, DT + t, e)];
      }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[slot_of(wave, t, e)] = dk[t][e];
        red[slot_of(wave, DT + t, e)] = dv[t][e];
      }
  }
  __syncthreads();
  const int key = k0 + l32;
  if (part >= 0) {  // a half: fp32 sums, unscaled, in [u][e][lane] order
    float* dst = a.dkv_part + ((int64_t)(bg * a.split + kb) * 2 + part) * (2 * DT * 16 * 64);
    for (int u = wave; u < 2 * DT; u += DKV_WAVES) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = red[slot_of(0, u, e)];
#pragma unroll
        for (int w = 1; w < 4; ++w) x += red[slot_of(w, u, e)];
        dst[(u * 16 + e) * 64 + lane] = x;
      }
    }
    return;
  }
  for (int u = wave; u < 2 * DT; u += DKV_WAVES) {
    const bool is_k = u < DT;
    const int dt = is_k ? u : u - DT;
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = red[slot_of(0, u, e)];
#pragma unroll
      for (int w = 1; w < 4; ++w) x += red[slot_of(w, u, e)];
      v[e] = is_k ? x * a.scale : x;
    }
    if (key < a.s) {
      uint16_t* dst = a.dqkv + (tok0 + key) * a.ld_qkv + (int64_t)(is_k ? a.q + g : a.q + a.kv + g) * D + 32 * dt;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float w4[4] = {v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
        Elem<uint16_t>::store4(dst + 8 * q4 + 4 * h, w4);
      }
    }
  }
}

// dK/dV of the split key blocks: the two halves added in a fixed order (first
// + second), dK scaled, stored as bf16.  One thread per (block, u, lane, q4):
// the four values 4 q4 .. 4 q4 + 3 of a lane's accumulator, i.e. four
// consecutive head dims of one key, as the whole-block path stores them.
template <int D>
__global__ void __launch_bounds__(NTHREADS) attn_bwd_dkv_combine_kernel(BwdArgs a) {
  constexpr int DT = D / 32, PART = 2 * DT * 16 * 64;
  const int64_t t = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  if (t >= (int64_t)a.b * a.kv * a.split * 2 * DT * 256) return;
  const int q4 = (int)(t & 3), lane = (int)((t >> 2) & 63);
  const int u = (int)((t >> 8) % (2 * DT));
  const int blk = (int)((t >> 8) / (2 * DT));  // bg * split + kb
  const int bg = blk / a.split, kb = blk % a.split;
  const int beta = bg / a.kv, g = bg % a.kv;
  const int key = kb * KEY_BLOCK + (lane & 31), h = lane >> 5;
  if (key >= a.s) return;
  const float* p0 = a.dkv_part + (int64_t)blk * 2 * PART + u * 16 * 64 + lane;
  const float* p1 = p0 + PART;
  const bool is_k = u < DT;
  const int dt = is_k ? u : u - DT;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = (4 * q4 + e) * 64;
    const float x = p0[r] + p1[r];
    v[e] = is_k ? x * a.scale : x;
  }
  uint16_t* dst = a.dqkv + ((int64_t)beta * a.s + key) * a.ld_qkv + (int64_t)(is_k ? a.q + g : a.q + a.kv + g) * D +
                  32 * dt + 8 * q4 + 4 * h;
  Elem<uint16_t>::store4(dst, v);
}

// ---- dQ ----------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(NTHREADS, 2) attn_bwd_dq_kernel(BwdArgs a, int hg) {
  constexpr int DT = D / 32, KK = D / 16;
  constexpr int TILE = DQ_KEYS * D * 2;  // one 64-key K or V tile
  constexpr int TI = TILE / 1024;
  constexpr int STAGE = 2 * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const lds_u8* lds = (const lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv;
  const int sub_per_kv = group / hg;
  const int ny = a.b * a.kv * sub_per_kv;
  int pb, y, part = -1, slot = -1;
  if (a.dq_split > 0)
    dq_job((int)blockIdx.x, npb, ny, a.dq_split, pb, y, part, slot);
  else
    attnt::causal_block_order(npb, ny, pb, y);
  const int beta = y / (a.kv * sub_per_kv);
  const int rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * hg + (wave % hg);
  const int pos0 = pb * rows_per_wg;
  const int rp0 = pos0 + (wave / hg) * 32;
  const int my_row = rp0 + l32;
  const int64_t tok0 = (int64_t)beta * a.s;
  const uint32_t ldq = (uint32_t)a.ld_qkv * 2u, ldo = (uint32_t)a.ld_o * 2u;

  // this lane's query row of Q and dO as MFMA operands, and its statistics
  bf16x8 qf[KK], of[KK];
  float lse2 = 0.0f, dlt = 0.0f;
  {
    const rsrc_t rq = make_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldq);
    const rsrc_t ro = make_rsrc(a.dO + tok0 * a.ld_o, (uint32_t)a.s * ldo);
    const bool ok = my_row < a.s;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint32_t c = (uint32_t)(j * D + 16 * kk + 8 * h) * 2u;
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, ok ? (uint32_t)my_row * ldq + c : kOOB));
      of[kk] = __builtin_bit_cast(bf16x8, buf_load16(ro, ok ? (uint32_t)my_row * ldo + c : kOOB));
    }
    if (ok) {
      const int64_t r = ((int64_t)beta * a.q + j) * a.s + my_row;
      lse2 = a.stats[2 * r];
      dlt = a.stats[2 * r + 1];
    }
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[t][e] = 0.0f;

  const int kv_end = a.causal ? min(a.s, pos0 + rows_per_wg) : a.s;
  const int nkb_all = (kv_end + DQ_KEYS - 1) / DQ_KEYS;
  // a half takes key blocks [kb0, kb0 + nkb)
  const int kb0 = part == 1 ? nkb_all / 2 : 0;
  const int nkb = part < 0 ? nkb_all : (part == 0 ? nkb_all / 2 : nkb_all - nkb_all / 2);
  const u32x4 rkv = lds::sgpr_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldq);
  const uint32_t kcol = (uint32_t)(a.q + g) * D * 2u, vcol = (uint32_t)(a.q + a.kv + g) * D * 2u;
  // every instruction i = wave + 4 p this wave issues has i = wave mod 4:
  // the per-lane part of its offsets is computed once
  const uint32_t kv_lane = attnt::dma_lane_off<D>(ldq, wave);
  auto issue = [&](int kb, int st) {
    const uint32_t dst = lds_base + (uint32_t)st * STAGE;
    const int row0 = (kb0 + kb) * DQ_KEYS;
#pragma unroll
    for (int i = wave; i < TI; i += 4) {
      attnt::dma_tile_part_at<D>(rkv, ldq, row0, kcol, dst, i, kv_lane);
      attnt::dma_tile_part_at<D>(rkv, ldq, row0, vcol, dst + TILE, i, kv_lane);
    }
  };
  if (nkb > 0) issue(0, 0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    lds::wait_vmcnt<0>();
    lds::wait_lgkm0();
    lds::barrier();  // block kb is in LDS for every wave; every wave is done with block kb-1
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    const int key0 = (kb0 + kb) * DQ_KEYS;
    if (a.causal && key0 > rp0 + 31) continue;
    const lds_u8* tk = lds + st * STAGE;
    const lds_u8* tv = tk + TILE;
    // blocks wholly inside the sequence and below the causal diagonal skip the mask
    const bool full = key0 + DQ_KEYS <= a.s && (!a.causal || key0 + DQ_KEYS - 1 <= rp0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // S^T = K Q^T and dP^T = V dO^T: lane = query, registers = keys
      f32x16 sacc, pacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = pacc[e] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(tk, 32 * kt, kk), qf[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(tv, 32 * kt, kk), of[kk], pacc, 0, 0, 0);
      }
      float ds[16];
      auto grads = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
          float p = __builtin_amdgcn_exp2f(sacc[r] * a.scale_log2 - lse2);
          if constexpr (decltype(masked)::value) {
            if (!(key < a.s && (!a.causal || key <= my_row))) p = 0.0f;
          }
          ds[r] = p * (pacc[r] - dlt);
        }
      };
      if (full)
        grads(std::false_type{});
      else
        grads(std::true_type{});
      const bf16x8 df0 = pack8(ds), df1 = pack8(ds + 8);
      // dQ^T += K^T dS^T: lane = query, registers = head dims; every d tile's
      // first product before any second one, so consecutive MFMAs do not
      // accumulate into the same registers
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tk, 32 * kt, dt, 0), df0, dq[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tk, 32 * kt, dt, 1), df1, dq[dt], 0, 0, 0);
    }
  }

  if (part >= 0) {  // a half: fp32 sums, unscaled, in [dt * 16 + e][lane] order
    float* dst = a.dq_part + ((int64_t)(slot * 2 + part) * 4 + wave) * (DT * 16 * 64);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(dt * 16 + e) * 64 + lane] = dq[dt][e];
    return;
  }
  if (my_row < a.s) {
    uint16_t* dst = a.dqkv + (tok0 + my_row) * a.ld_qkv + (int64_t)j * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float w4[4] = {dq[dt][4 * q4] * a.scale, dq[dt][4 * q4 + 1] * a.scale, dq[dt][4 * q4 + 2] * a.scale,
                             dq[dt][4 * q4 + 3] * a.scale};
        Elem<uint16_t>::store4(dst + 32 * dt + 8 * q4 + 4 * h, w4);
      }
  }
}

// dQ from the dS tiles handed over by dK/dV (BwdArgs::ds_path): nothing of
// the scores, dP or the exponentials is recomputed.  Work-groups, waves and
// block order as attn_bwd_dq_kernel; per 64-key block a wave of 32 query rows
// (query tile qt) takes the block's K rows (shared in LDS, double buffered,
// LDS-direct loads) and its own two 32 x 32 dS tiles (the key halves
// kb <= qt), loaded a block ahead straight into registers in the image its
// products take, and adds dQ^T += K^T dS^T in the order of
// attn_bwd_dq_kernel's products.
template <int D>
__global__ void __launch_bounds__(NTHREADS, 2) attn_bwd_dq_ds_kernel(BwdArgs a, int hg) {
  constexpr int DT = D / 32;
  constexpr int TILE = DQ_KEYS * D * 2;  // one 64-key K tile
  constexpr int TI = TILE / 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * TILE];
  const lds_u8* lds = (const lds_u8*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv;
  const int sub_per_kv = group / hg;
  const int ny = a.b * a.kv * sub_per_kv;
  int pb, y;
  attnt::causal_block_order(npb, ny, pb, y);
  const int beta = y / (a.kv * sub_per_kv);
  const int rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * hg + (wave % hg);
  const int pos0 = pb * rows_per_wg;
  const int rp0 = pos0 + (wave / hg) * 32;
  const int qt = rp0 / 32;
  const int my_row = rp0 + l32;
  const int64_t tok0 = (int64_t)beta * a.s;
  const uint32_t ldq = (uint32_t)a.ld_qkv * 2u;
  const int nqt = (a.s + 31) / 32;
  const int64_t tile0 = ((int64_t)beta * a.q + j) * ((int64_t)nqt * (nqt + 1) / 2) + (int64_t)qt * (qt + 1) / 2;
  const int64_t tiles_all = (int64_t)a.b * a.q * ((int64_t)nqt * (nqt + 1) / 2);
  const u32x4 rkv = lds::sgpr_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldq);
  const rsrc_t rda = make_rsrc(a.ds_a, (uint32_t)(a.ds_t0 * 2048));
  const rsrc_t rdb = make_rsrc(a.ds_b, (uint32_t)(tiles_all > a.ds_t0 ? (tiles_all - a.ds_t0) * 2048 : 0));
  const uint32_t kcol = (uint32_t)(a.q + g) * D * 2u;

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[t][e] = 0.0f;

  const int kv_end = min(a.s, pos0 + rows_per_wg);
  const int nkb = (kv_end + DQ_KEYS - 1) / DQ_KEYS;
  // every K instruction i = wave + 4 p this wave issues has i = wave mod 4:
  // the per-lane part of its offsets is computed once
  const uint32_t kv_lane = attnt::dma_lane_off<D>(ldq, wave);
  auto issue_k = [&](int kb) {
    const uint32_t dst = lds_base + (uint32_t)(kb & 1) * TILE;
#pragma unroll
    for (int i = wave; i < TI; i += 4) attnt::dma_tile_part_at<D>(rkv, ldq, kb * DQ_KEYS, kcol, dst, i, kv_lane);
  };
  // a block's two dS tiles, [kt][jj] (halves past the causal range or past
  // the last block read zeros)
  struct DsRegs {
    bf16x8 f[2][2];
  };
  auto load_ds = [&](int kb, DsRegs& r) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kb32 = 2 * kb + kt;
      const int64_t t = tile0 + kb32;
      const bool ok = kb < nkb && kb32 <= qt;
      const bool in_a = t < a.ds_t0;
      const uint32_t off = ok ? (uint32_t)((in_a ? t : t - a.ds_t0) * 2048) + (uint32_t)lane * 16u : kOOB;
      const rsrc_t rd = in_a ? rda : rdb;
      r.f[kt][0] = __builtin_bit_cast(bf16x8, buf_load16(rd, off));
      r.f[kt][1] = __builtin_bit_cast(bf16x8, buf_load16(rd, ok ? off + 1024u : kOOB));
    }
  };
  DsRegs R[2];
  if (nkb > 0) {
    load_ds(0, R[0]);
    issue_k(0);
  }
  for (int kb0 = 0; kb0 < nkb; kb0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = kb0 + u;
      if (kb >= nkb) break;
      // K of block kb and this wave's dS of block kb have landed
      lds::wait_vmcnt<0>();
      lds::wait_lgkm0();
      lds::barrier();  // block kb's K is in LDS for every wave; every wave is done with block kb-1
      load_ds(kb + 1, R[(u + 1) % 2]);
      if (kb + 1 < nkb) issue_k(kb + 1);
      const lds_u8* tk = lds + (kb & 1) * TILE;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (2 * kb + kt > qt) break;
        const bf16x8 df0 = R[u].f[kt][0], df1 = R[u].f[kt][1];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tk, 32 * kt, dt, 0), df0, dq[dt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(tk, 32 * kt, dt, 1), df1, dq[dt], 0, 0, 0);
      }
    }
  }
  lds::wait_vmcnt<0>();  // no load into LDS outlives the work-group
  if (my_row < a.s) {
    uint16_t* dst = a.dqkv + (tok0 + my_row) * a.ld_qkv + (int64_t)j * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float w4[4] = {dq[dt][4 * q4] * a.scale, dq[dt][4 * q4 + 1] * a.scale, dq[dt][4 * q4 + 2] * a.scale,
                             dq[dt][4 * q4 + 3] * a.scale};
        Elem<uint16_t>::store4(dst + 32 * dt + 8 * q4 + 4 * h, w4);
      }
  }
}

// dQ of the split query blocks: the two halves added in a fixed order (first
// + second), scaled and stored as bf16, with the row and head mapping of
// attn_bwd_dq_kernel.  One thread per (slot, wave, dt, lane), the lane
// fastest so that every load reads 64 consecutive floats.
template <int D>
__global__ void __launch_bounds__(NTHREADS) attn_bwd_dq_combine_kernel(BwdArgs a, int hg) {
  constexpr int DT = D / 32, PART = 4 * DT * 16 * 64;
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int group = a.q / a.kv, sub_per_kv = group / hg;
  const int ny = a.b * a.kv * sub_per_kv;
  const int64_t t = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  if (t >= (int64_t)a.dq_split * ny * 4 * 64 * DT) return;
  const int lane = (int)(t & 63), dt = (int)((t >> 6) % DT), wave = (int)(((t >> 6) / DT) & 3);
  const int slot = (int)((t >> 6) / DT / 4);
  const int i = slot / ny, y = slot % ny;
  const int pb = npb - 1 - i;
  const int beta = y / (a.kv * sub_per_kv), rem = y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * hg + (wave % hg);
  const int my_row = pb * rows_per_wg + (wave / hg) * 32 + (lane & 31), h = lane >> 5;
  if (my_row >= a.s) return;
  const float* p0 = a.dq_part + ((int64_t)(slot * 2) * 4 + wave) * (DT * 16 * 64) + dt * 16 * 64 + lane;
  const float* p1 = p0 + PART;
  uint16_t* dst = a.dqkv + ((int64_t)beta * a.s + my_row) * a.ld_qkv + (int64_t)j * D + 32 * dt + 4 * h;
  float x0[16], x1[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    x0[e] = p0[e * 64];
    x1[e] = p1[e * 64];
  }
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (x0[4 * q4 + e] + x1[4 * q4 + e]) * a.scale;
    Elem<uint16_t>::store4(dst + 8 * q4, v);
  }
}

}  // namespace attnb

template <int D>
hipError_t launch_attn_bwd_stats(const attnb::BwdArgs& a, hipStream_t stream) {
  const int64_t nrows = (int64_t)a.b * a.q * a.s;
  if (nrows == 0) return hipSuccess;
  constexpr int RPB = attnb::NTHREADS / (D / 8) * attnb::STATS_ROWS;
  tp_launch((attnb::attn_bwd_stats_kernel<D>), dim3((unsigned)((nrows + RPB - 1) / RPB)),
            dim3(attnb::NTHREADS), 0, stream, a, nrows);
  return hipGetLastError();
}

// Key blocks worth splitting (see BwdArgs::split): all but the lightest
// eighth for a causal mask (a model of the in-order dispatch of the jobs,
// heaviest first, gives the shortest kernel there), none otherwise (every
// block then sees every query).
inline int attn_bwd_dkv_split(int s, int causal) {
  const int nkb = (s + attnb::KEY_BLOCK - 1) / attnb::KEY_BLOCK;
  return causal ? nkb - nkb / 8 : 0;
}
// Floats of dkv_part for `split` split key blocks.
inline int64_t attn_bwd_dkv_part_floats(int b, int kv, int split, int d) {
  return (int64_t)b * kv * split * 2 * (2 * (d / 32) * 16 * 64);
}

// dK/dV (a.split and a.dkv_part set by the caller; split <= nkb), then the
// kernel that finishes the split blocks.
template <int D>
hipError_t launch_attn_bwd_dkv(const attnb::BwdArgs& a, hipStream_t stream) {
  const int nkb = (a.s + attnb::KEY_BLOCK - 1) / attnb::KEY_BLOCK;
  const int BG = a.b * a.kv;
  if (nkb == 0 || BG == 0) return hipSuccess;
  tp_launch((attnb::attn_bwd_dkv_kernel<D>), dim3(BG * (nkb + a.split)), dim3(64 * attnb::DKV_WAVES), 0,
            stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split == 0) return e;
  const int64_t n = (int64_t)BG * a.split * 2 * (D / 32) * 256;
  tp_launch((attnb::attn_bwd_dkv_combine_kernel<D>), dim3((unsigned)((n + attnb::NTHREADS - 1) / attnb::NTHREADS)),
            dim3(attnb::NTHREADS), 0, stream, a);
  return hipGetLastError();
}

// Query blocks of the dQ launch worth splitting (BwdArgs::dq_split): the
// heavier half for a causal mask when the unsplit launch leaves some of the
// 512 work-group slots (two per CU) empty, none otherwise (with every slot
// taken, the heavy-light pairing of causal_block_order measured faster than
// the split); and the floats of dq_part.
inline int attn_bwd_dq_split(int s, int causal, int b, int q, int kv, int hg) {
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (s + rows_per_wg - 1) / rows_per_wg;
  const int64_t wgs = (int64_t)npb * b * kv * ((q / kv) / hg);
  return causal && wgs < 512 ? npb / 2 : 0;
}
inline int64_t attn_bwd_dq_part_floats(int b, int q, int kv, int hg, int dq_split, int d) {
  return (int64_t)dq_split * b * kv * ((q / kv) / hg) * 2 * 4 * (d / 32) * 16 * 64;
}

// dQ: from the handed-over dS tiles when a.ds_path, else recomputing the
// scores (a.dq_split and a.dq_part set by the caller; dq_split <= npb / 2),
// then the kernel that finishes the split blocks.
template <int D>
hipError_t launch_attn_bwd_dq(const attnb::BwdArgs& a, int hg, hipStream_t stream) {
  const int rows_per_wg = 32 * (4 / hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int ny = a.b * a.kv * ((a.q / a.kv) / hg);
  if (npb == 0 || ny == 0) return hipSuccess;
  if (a.ds_path) {
    tp_launch((attnb::attn_bwd_dq_ds_kernel<D>), dim3(npb, ny), dim3(attnb::NTHREADS), 0, stream, a, hg);
    return hipGetLastError();
  }
  if (a.dq_split == 0) {
    tp_launch((attnb::attn_bwd_dq_kernel<D>), dim3(npb, ny), dim3(attnb::NTHREADS), 0, stream, a, hg);
    return hipGetLastError();
  }
  tp_launch((attnb::attn_bwd_dq_kernel<D>), dim3((npb + a.dq_split) * ny), dim3(attnb::NTHREADS), 0, stream,
            a, hg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)a.dq_split * ny * 4 * 64 * (D / 32);
  tp_launch((attnb::attn_bwd_dq_combine_kernel<D>), dim3((unsigned)((n + attnb::NTHREADS - 1) / attnb::NTHREADS)),
            dim3(attnb::NTHREADS), 0, stream, a, hg);
  return hipGetLastError();
}

}  // namespace tp
