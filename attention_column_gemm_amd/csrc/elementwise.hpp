// HBM-bound kernels of the shard: the emulated all-reduce (rank-ordered sum
// of partials, bias once, dropout, residual), the same fused with the
// token-wise norm of each row, the all-gather copy, dropout backward, and
// deterministic column sums for the bias gradients.
//
// They stream 16-byte vectors (8 bf16 or 4 fp32) and do no reuse, so their
// roofline is HBM bandwidth.
#pragma once

#include "common.hpp"

namespace tp {

constexpr int MAX_PARTIALS = 64;
struct PartialPtrs {
  const void* p[MAX_PARTIALS];
};

// 16-byte load of data read once, with the sc1 cache policy, through a buffer
// descriptor based at `base` (so that 32-bit offsets suffice): measured about
// 15% faster than plain loads for the partial sums' streams on gfx950.
__device__ __forceinline__ u32x4 load_once16(const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(base, 0xffffffffu), byte_off, 0, 2 /* sc1 */);
}

template <class T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4& w, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16lo(w[i]); v[2 * i + 1] = bf16hi(w[i]); }
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[8]) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16lo(w[i]); v[2 * i + 1] = bf16hi(w[i]); }
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
  // the values as store() writes them (round to nearest even), back in fp32
  __device__ __forceinline__ static void round(const float (&v)[8], float (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      r[2 * i] = bf16lo(w);
      r[2 * i + 1] = bf16hi(w);
    }
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4& w, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ static void load(const float* p, float (&v)[4]) {
    f32x4 w = *reinterpret_cast<const f32x4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
  __device__ __forceinline__ static void round(const float (&v)[4], float (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i];
  }
};

// out = residual + Dropout(sum_{i<t} P_i + bias).  The partials are summed
// in rank order in fp32; the bias is added once, after the sum; the dropout
// decision of the element at flat index e of this call's range comes from
// dropout_keep(seed, idx0 + e, thr), idx0 being the range's first index in
// the full tensor (so a token slice keeps the full tensor's mask); the
// residual (optional) is added last.  cols is a multiple of the vector width,
// so one vector lies in one row.
template <class T>
__global__ void __launch_bounds__(256) sum_partials_kernel(int64_t n_vec, int64_t cols, int t, PartialPtrs P,
                                                           const T* __restrict__ bias, uint32_t thr, float scale,
                                                           uint64_t seed, uint64_t idx0,
                                                           const T* __restrict__ residual, T* __restrict__ out) {
  constexpr int V = Vec<T>::N;
  // block-uniform chunk starts keep the descriptors' bases scalar
  for (int64_t v0 = (int64_t)blockIdx.x * blockDim.x; v0 < n_vec; v0 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = v0 + threadIdx.x;
    if (v >= n_vec) break;
    const int64_t e0 = v * V;
    const uint32_t off = threadIdx.x * 16u;
    float acc[V];
    for (int i0 = 0; i0 < t; i0 += 8) {  // up to eight partials' loads in flight, summed in rank order
      const int nb = t - i0 < 8 ? t - i0 : 8;
      u32x4 w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k < nb) w[k] = load_once16(reinterpret_cast<const T*>(P.p[i0 + k]) + v0 * V, off);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k >= nb) break;
        float x[V];
        Vec<T>::unpack(w[k], x);
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] = (i0 + k == 0) ? x[j] : acc[j] + x[j];
      }
    }
    if (bias) {
      float b[V];
      Vec<T>::load(bias + (e0 % cols), b);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += b[j];
    }
    if (thr) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        acc[j] = dropout_keep(seed, idx0 + (uint64_t)(e0 + j), thr) ? acc[j] * scale : 0.0f;
    }
    if (residual) {
      float r[V];
      Vec<T>::unpack(load_once16(residual + v0 * V, off), r);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += r[j];
    }
    Vec<T>::store(out + e0, acc);
  }
}

// Sum of a block's 256 threads' values in a fixed order: a butterfly within
// each wave, then the four wave sums in wave order (every thread gets the
// same bits).  `red` holds four floats of LDS; the caller separates two uses
// of it with a barrier.
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Block output and its token-wise norm, one row per work-group of 256
// threads.  Row r of this call (global row row0 + r):
//   out    = residual + Dropout(sum_{i<t} P_i + bias)     (as sum_partials_kernel)
//   normed = norm(out as stored), RMSNorm x / sqrt(mean(x^2) + eps) * gamma
//            or LayerNorm (x - mean) / sqrt(var + eps) * gamma + beta.
// Thread j owns vectors j, j + 256, ... of the row (NV of them at most), so
// the row stays in registers between the sum and the norm; the statistics
// are fp32 sums in a fixed order (LayerNorm's variance from the mean-free
// values).  The partials' pointers are already offset to row0.
template <class T, int NV>
__global__ void __launch_bounds__(256) sum_norm_kernel(int64_t cols, int t, PartialPtrs P, const T* __restrict__ bias,
                                                       uint32_t thr, float scale, uint64_t seed, uint64_t idx0,
                                                       const T* __restrict__ residual, int layer_norm,
                                                       const T* __restrict__ gamma, const T* __restrict__ beta,
                                                       float eps, T* __restrict__ out, T* __restrict__ normed) {
  constexpr int V = Vec<T>::N;
  __shared__ float red[2][4];
  const int64_t r = blockIdx.x;
  const int nvec = (int)(cols / V);
  const int64_t row_off = r * cols;  // elements
  float x[NV][V];
  float s1 = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = (int)threadIdx.x + i * 256;
#pragma unroll
    for (int j = 0; j < V; ++j) x[i][j] = 0.0f;
    if (v >= nvec) continue;
    const int64_t e0 = row_off + (int64_t)v * V;
    const uint32_t off = (uint32_t)v * 16u;
    float acc[V];
    for (int i0 = 0; i0 < t; i0 += 8) {  // up to eight partials' loads in flight, summed in rank order
      const int nb = t - i0 < 8 ? t - i0 : 8;
      u32x4 w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k < nb) w[k] = load_once16(reinterpret_cast<const T*>(P.p[i0 + k]) + row_off, off);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k >= nb) break;
        float y[V];
        Vec<T>::unpack(w[k], y);
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] = (i0 + k == 0) ? y[j] : acc[j] + y[j];
      }
    }
    if (bias) {
      float b[V];
      Vec<T>::load(bias + (int64_t)v * V, b);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += b[j];
    }
    if (thr) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        acc[j] = dropout_keep(seed, idx0 + (uint64_t)(e0 + j), thr) ? acc[j] * scale : 0.0f;
    }
    if (residual) {
      float y[V];
      Vec<T>::unpack(load_once16(residual + row_off, off), y);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += y[j];
    }
    // store, and keep the value as stored (rounded to the storage type)
    Vec<T>::store(out + e0, acc);
    Vec<T>::round(acc, x[i]);
#pragma unroll
    for (int j = 0; j < V; ++j) s1 += x[i][j];
  }
  const float inv_n = 1.0f / (float)cols;
  float mean = 0.0f;
  if (layer_norm) {
    mean = block_sum256(s1, red[0]) * inv_n;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if ((int)threadIdx.x + i * 256 < nvec)
#pragma unroll
        for (int j = 0; j < V; ++j) x[i][j] -= mean;
  }
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < V; ++j) s2 += x[i][j] * x[i][j];
  const float rstd = __builtin_amdgcn_rsqf(block_sum256(s2, red[1]) * inv_n + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = (int)threadIdx.x + i * 256;
    if (v >= nvec) continue;
    float g[V], y[V];
    if (gamma) Vec<T>::load(gamma + (int64_t)v * V, g);
    else
#pragma unroll
      for (int j = 0; j < V; ++j) g[j] = 1.0f;
#pragma unroll
    for (int j = 0; j < V; ++j) y[j] = x[i][j] * rstd * g[j];
    if (beta) {
      float b[V];
      Vec<T>::load(beta + (int64_t)v * V, b);
#pragma unroll
      for (int j = 0; j < V; ++j) y[j] += b[j];
    }
    Vec<T>::store(normed + row_off + (int64_t)v * V, y);
  }
}

// out = [S_0; S_1; ...; S_{t-1}]: the t slices of n_vec_slice vectors each,
// concatenated in rank order (16-byte vector copies).
__global__ void __launch_bounds__(256) gather_kernel(int64_t n_vec_slice, int t, PartialPtrs S, u32x4* __restrict__ out) {
  const int64_t n = n_vec_slice * t;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / n_vec_slice, e = v - r * n_vec_slice;
    out[v] = reinterpret_cast<const u32x4*>(S.p[r])[e];
  }
}

// dY = dOut * keep / (1 - p)  (thr = 0: plain copy).
template <class T>
__global__ void __launch_bounds__(256) dropout_bwd_kernel(int64_t n_vec, const T* __restrict__ dOut, uint32_t thr,
                                                          float scale, uint64_t seed, T* __restrict__ dY) {
  constexpr int V = Vec<T>::N;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n_vec; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = v * V;
    float x[V];
    Vec<T>::load(dOut + e0, x);
    if (thr) {
#pragma unroll
      for (int j = 0; j < V; ++j) x[j] = dropout_keep(seed, (uint64_t)(e0 + j), thr) ? x[j] * scale : 0.0f;
    }
    Vec<T>::store(dY + e0, x);
  }
}

// out[c] = sum over rows of X[r, c] in fp32, in a fixed order (so repeated
// runs agree bit for bit).  A work-group owns CV column vectors (CV * V
// columns): its 256 threads are CV column vectors x 256/CV row lanes; lane l
// sums rows l, l + ROW_LANES, ... in that order (four loads in flight), and
// the lanes are then folded pairwise through LDS.  The launcher picks CV so
// that narrow tensors still spread over the CUs.
template <class T, int CV>
__global__ void __launch_bounds__(256) colsum_kernel(int64_t rows, int64_t cols, int64_t ld, const T* __restrict__ X,
                                                     float* __restrict__ out) {
  constexpr int V = Vec<T>::N;
  constexpr int ROW_LANES = 256 / CV;
  __shared__ float red[ROW_LANES][CV * V + 1];
  const int cv = threadIdx.x % CV, rl = threadIdx.x / CV;
  const int64_t c0 = (int64_t)blockIdx.x * CV * V + cv * V;
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.0f;
  if (c0 < cols) {
    int64_t r = rl;
    for (; r + 3 * ROW_LANES < rows; r += 4 * ROW_LANES) {
      float x[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) Vec<T>::load(X + (r + u * ROW_LANES) * ld + c0, x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] += x[u][j];
    }
    for (; r < rows; r += ROW_LANES) {
      float x[V];
      Vec<T>::load(X + r * ld + c0, x);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += x[j];
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) red[rl][cv * V + j] = acc[j];
  __syncthreads();
  for (int s = ROW_LANES / 2; s > 0; s >>= 1) {
    if (rl < s) {
#pragma unroll
      for (int j = 0; j < V; ++j) red[rl][cv * V + j] += red[rl + s][cv * V + j];
    }
    __syncthreads();
  }
  if (rl == 0 && c0 < cols) {
#pragma unroll
    for (int j = 0; j < V; ++j) out[c0 + j] = red[0][cv * V + j];
  }
}

}  // namespace tp
