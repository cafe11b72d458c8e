// fp32 GEMM on the vector ALUs, for shards stored in fp32 end to end.
//
// Same problem description and epilogues as the bf16 matrix-core GEMM
// (GemmProblem with float pointers reinterpreted), so an fp32 shard runs the
// same sequence of fused steps; it never rounds to a narrower type.  Sized for
// small shards: 64x64 block tile, K step 16, 256 threads each owning a 4x4
// micro-tile of four consecutive columns.
#pragma once

#include "common.hpp"
#include "gemm_common.hpp"

namespace tp {
namespace simt {

constexpr int BM = 64, BN = 64, BK = 16, NTHREADS = 256;

template <int LAYOUT>
__device__ __forceinline__ float load_op(const float* __restrict__ g, int64_t ld, int row, int k, int nrows, int K) {
  if (row >= nrows || k >= K) return 0.0f;
  return LAYOUT == KMAJOR ? g[(int64_t)row * ld + k] : g[(int64_t)k * ld + row];
}

template <int AL, int BL, class Epi>
__global__ void __launch_bounds__(NTHREADS) gemm_f32_kernel(GemmProblem p, Epi epi) {
  constexpr int NB = Epi::NB;
  __shared__ float As[BK][BM];
  __shared__ float Bs[NB][BK][BN];
  const int tiles_n = (p.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[NB][4][4] = {};
  for (int s = 0; s < p.nseg; ++s) {
    const float* A = reinterpret_cast<const float*>(p.A[s]);
    for (int k0 = 0; k0 < p.K[s]; k0 += BK) {
      // 64x16 elements per operand, 4 per thread
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + NTHREADS * i;
        const int kk = e % BK, rr = e / BK;
        As[kk][rr] = load_op<AL>(A, p.lda[s], m0 + rr, k0 + kk, p.M, p.K[s]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          Bs[b][kk][rr] = load_op<BL>(reinterpret_cast<const float*>(p.B[s][b]), p.ldb[s], n0 + rr, k0 + kk, p.N, p.K[s]);
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float bv = Bs[b][kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[b][i][j] = fmaf(a[i], bv, acc[b][i][j]);
          }
      }
      __syncthreads();
    }
  }
  typename Epi::Aux aux[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) epi.load(m0 + ty * 4 + i, n0 + tx * 4, aux[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[b][j] = acc[b][i][j];
    epi(m0 + ty * 4 + i, n0 + tx * 4, v, aux[i]);
  }
}

}  // namespace simt

template <int AL, int BL, class Epi>
hipError_t launch_gemm_f32(const GemmProblem& p, const Epi& epi, hipStream_t stream) {
  const int tiles = ((p.M + simt::BM - 1) / simt::BM) * ((p.N + simt::BN - 1) / simt::BN);
  if (tiles == 0) return hipSuccess;
  tp_launch((simt::gemm_f32_kernel<AL, BL, Epi>), dim3(tiles), dim3(simt::NTHREADS), 0, stream, p, epi);
  return hipGetLastError();
}

}  // namespace tp
