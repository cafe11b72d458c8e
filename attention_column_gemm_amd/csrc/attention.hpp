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
//  * Keys advance in blocks of 64.  S^T = K Q^T is formed with
//    v_mfma_f32_32x32x16_bf16 taking the K fragment as first operand, which
//    leaves one query row per lane (its 64 keys split between lanes l and
//    l + 32): row maxima need one cross-half exchange, and the running sums
//    stay per lane until the end.
//  * O^T = V^T P^T uses the probabilities straight from the S registers as the
//    second operand; the K index order of that MFMA is permuted to match the
//    accumulator layout, and V is staged transposed ([d][key]) in LDS in the
//    same permuted order, so P never goes through LDS.
//  * Online softmax in base 2 (scores pre-multiplied by log2(e)/sqrt(d)).
//  * K/V blocks are double buffered; work-groups are issued heaviest-first
//    (latest query rows) to even out the causal triangle.
#pragma once

#include "common.hpp"

namespace tp {
namespace attn {

constexpr int BKV = 64;
constexpr int NTHREADS = 256;

struct AttnArgs {
  const uint16_t* qkv;   // [T, (q + 2kv) d]
  uint16_t* o;           // [T, q d]
  float* lse;            // [b, q, s] or null
  int64_t ld_qkv, ld_o;
  int b, s, q, kv, hg;   // hg: query heads per work-group
  int causal;
  float scale_log2;      // log2(e) / sqrt(d)
};

template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {  // K tile [64][D], D/8 chunks per row
  return row * D + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ int vt_off(int row, int chunk) {  // V^T tile [D][64], 8 chunks per row
  // rows are written 8 apart by the transposing loader and read 8 consecutive
  // at a time, so the swizzle mixes bits 0-2 and 3-5 of the row
  return row * BKV + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 3);
}

template <int D>
__global__ void __launch_bounds__(NTHREADS, 1) attn_fwd_kernel(AttnArgs a) {
  constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  constexpr int KPER = BKV * KCH / NTHREADS; // K chunks per thread
  constexpr int DT = D / 32;                 // 32-wide d tiles of O
  constexpr int KK = D / 16;                 // k steps of S = Q K^T
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * BKV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int hgrp = lane >> 5, l32 = lane & 31;
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int pb = npb - 1 - (int)blockIdx.x;
  const int group = a.q / a.kv;
  const int sub_per_kv = group / a.hg;
  const int beta = blockIdx.y / (a.kv * sub_per_kv);
  const int rem = blockIdx.y % (a.kv * sub_per_kv);
  const int g = rem / sub_per_kv;
  const int j = g * group + (rem % sub_per_kv) * a.hg + (wave % a.hg);
  const int pos0 = pb * rows_per_wg;
  const int rp0 = pos0 + (wave / a.hg) * 32;
  const int my_row = rp0 + l32;
  const int64_t tok0 = (int64_t)beta * a.s;

  // Q fragments of this lane's row (zero beyond the sequence).
  bf16x8 qf[KK];
  {
    const uint16_t* qrow = a.qkv + (tok0 + my_row) * a.ld_qkv + (int64_t)j * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = {0, 0, 0, 0};
      if (my_row < a.s) w = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hgrp * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kv_end = a.causal ? min(a.s, pos0 + rows_per_wg) : a.s;
  const int nkb = (kv_end + BKV - 1) / BKV;
  // this sequence's rows of QKV behind a buffer resource (zeros past its end)
  const uint32_t ldb = (uint32_t)a.ld_qkv * 2u;
  const rsrc_t seq = make_rsrc(a.qkv + tok0 * a.ld_qkv, (uint32_t)a.s * ldb);
  const uint32_t kcol = (uint32_t)(a.q + g) * D * 2u, vcol = (uint32_t)(a.q + a.kv + g) * D * 2u;

  u32x4 kreg[KPER];
  u32x4 vreg[8];
  auto issue = [&](int kb) {
    const int key0 = kb * BKV;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int c = tid + NTHREADS * i;
      const int row = c / KCH, ch = c % KCH;
      kreg[i] = buf_load16(seq, key0 + row < a.s ? (uint32_t)(key0 + row) * ldb + kcol + ch * 16u : kOOB);
    }
    if (tid < D) {  // D blocks of 8 keys x 8 dims
      const int dg = tid % KCH, kg = tid / KCH;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int key = key0 + kg * 8 + r;
        vreg[r] = buf_load16(seq, key < a.s ? (uint32_t)key * ldb + vcol + dg * 16u : kOOB);
      }
    }
  };
  auto commit = [&](int st) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int c = tid + NTHREADS * i;
      *reinterpret_cast<u32x4*>(&Ks[st][k_off<D>(c / KCH, c % KCH)]) = kreg[i];
    }
    if (tid < D) {
      const int dg = tid % KCH, kg = tid / KCH;
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // dim dg*8 + i, keys kg*8 .. kg*8+7
        u32x4 w;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t lo = vreg[2 * q2][i >> 1], hi = vreg[2 * q2 + 1][i >> 1];
          w[q2] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<u32x4*>(&Vt[st][vt_off(dg * 8 + i, kg)]) = w;
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (nkb > 0) {
    issue(0);
    commit(0);
  }
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nkb) issue(kb + 1);
    const int key0 = kb * BKV;
    const bool active = !a.causal || key0 <= rp0 + 31;
    if (active) {
      // S^T for two 32-key tiles
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[st][k_off<D>(kt * 32 + l32, kk * 2 + hgrp)]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kt], 0, 0, 0);
        }
      }
      // scale, mask, block max
      const bool need_mask = (a.causal && key0 + BKV - 1 > rp0) || key0 + BKV > a.s;
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kt][r] * a.scale_log2;
          if (need_mask) {
            const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hgrp + (r & 3);
            if (key >= a.s || (a.causal && key > my_row)) x = -INFINITY;
          }
          sacc[kt][r] = x;
          bmax = fmaxf(bmax, x);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run, bmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.0f;
      bf16x8 pf[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = exp2f(sacc[kt][8 * half + 2 * e] - m_use);
            const float p1 = exp2f(sacc[kt][8 * half + 2 * e + 1] - m_use);
            psum += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          u32x4 wv = {w[0], w[1], w[2], w[3]};
          pf[kt * 2 + half] = __builtin_bit_cast(bf16x8, wv);
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;
      // O^T += V^T P^T; k step jj covers keys 32*(jj/2) + 16*(jj%2) + {4*hgrp+i, 8+4*hgrp+i}
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kfirst = 32 * (jj >> 1) + 16 * (jj & 1) + 4 * hgrp;
        const int c0 = kfirst >> 3, h0 = (kfirst & 7) >> 2;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const int row = t * 32 + l32;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(&Vt[st][vt_off(row, c0) + h0 * 4]);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(&Vt[st][vt_off(row, c0 + 1) + h0 * 4]);
          const u32x4 vv = {lo.x, lo.y, hi.x, hi.y};
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[jj], oacc[t], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) commit(st ^ 1);
    __syncthreads();
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

}  // namespace attn

template <int D>
hipError_t launch_attn_fwd(const attn::AttnArgs& a, hipStream_t stream) {
  const int rows_per_wg = 32 * (4 / a.hg);
  const int npb = (a.s + rows_per_wg - 1) / rows_per_wg;
  const int ny = a.b * a.kv * ((a.q / a.kv) / a.hg);
  if (npb == 0 || ny == 0) return hipSuccess;
  hipLaunchKernelGGL((attn::attn_fwd_kernel<D>), dim3(npb, ny), dim3(attn::NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tp
