// GEMM epilogues: what happens to an fp32 accumulator tile before it leaves
// the registers.  Every epilogue is called with one row m and four consecutive
// columns n..n+3 (n a multiple of 4, N a multiple of 4) and the NB accumulator
// values of those columns, one set per B operand.
//
// Epilogues that read saved tensors (the backward ones) do so in two phases:
// load(m, n, aux) issues the reads into an Aux record, and the call operator
// consumes it.  The GEMM kernels issue the loads of many (m, n) groups before
// consuming any, so the memory latency is paid once per batch rather than once
// per group.
//
// The fusions follow where the pages put the elementwise work of an MLP shard:
// the activation (GeLU or SwiGLU's SiLU-gated product) runs locally on the
// column-parallel GEMM's output columns ([L11] section 2 -- "[L11]" is the
// grasp.study lesson "张量并行线性层分片与前反向通信量计算"; [TP1] "Tensor
// Parallelism张量并行（一）", column split), and its backward runs locally on
// the same columns when the row-parallel layer's input gradient is formed
// ([L11] section 3, backward list).
#pragma once

#include "common.hpp"

namespace tp {

// C[m, n] = acc   (partials Z_i and dX_i, QKV, attention output projection, weight gradients)
template <class T>
struct EpiStore {
  static constexpr int NB = 1;
  struct Aux {};
  T* C;
  int64_t ldc;
  int M, N;
  __device__ __forceinline__ void load(int, int, Aux&) const {}
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& = Aux()) const {
    if (m >= M || n >= N) return;
    Elem<T>::store4(C + (int64_t)m * ldc + n, v[0]);
  }
};

// Two B operands sharing A: C0 = A B0, C1 = A B1 (SwiGLU weight gradients dWg_i, dWu_i).
template <class T>
struct EpiStore2 {
  static constexpr int NB = 2;
  struct Aux {};
  T* C0;
  T* C1;
  int64_t ldc;
  int M, N;
  __device__ __forceinline__ void load(int, int, Aux&) const {}
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& = Aux()) const {
    if (m >= M || n >= N) return;
    Elem<T>::store4(C0 + (int64_t)m * ldc + n, v[0]);
    Elem<T>::store4(C1 + (int64_t)m * ldc + n, v[1]);
  }
};

// GeLU forward: A = acc + b1 (b1 may be null), H = GeLU(A); both stored.
template <class T>
struct EpiGeluFwd {
  static constexpr int NB = 1;
  struct Aux {};
  T* A;
  T* H;
  const T* b1;
  int64_t ld;
  int M, N;
  __device__ __forceinline__ void load(int, int, Aux&) const {}
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& = Aux()) const {
    if (m >= M || n >= N) return;
    float a[4] = {v[0][0], v[0][1], v[0][2], v[0][3]};
    if (b1) {
      float b[4];
      Elem<T>::load4(b1 + n, b);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] += b[j];
    }
    float hv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hv[j] = gelu_f(a[j]);
    Elem<T>::store4(A + (int64_t)m * ld + n, a);
    Elem<T>::store4(H + (int64_t)m * ld + n, hv);
  }
};

// SwiGLU forward: G = acc0 (gate), U = acc1 (up), H = SiLU(G) * U; all stored.
template <class T>
struct EpiSwigluFwd {
  static constexpr int NB = 2;
  struct Aux {};
  T* G;
  T* U;
  T* H;
  int64_t ld;
  int M, N;
  __device__ __forceinline__ void load(int, int, Aux&) const {}
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& = Aux()) const {
    if (m >= M || n >= N) return;
    float hv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hv[j] = silu_f(v[0][j]) * v[1][j];
    const int64_t o = (int64_t)m * ld + n;
    Elem<T>::store4(G + o, v[0]);
    Elem<T>::store4(U + o, v[1]);
    Elem<T>::store4(H + o, hv);
  }
};

// GeLU backward: acc = dH; dA = dH * GeLU'(A_saved).
template <class T>
struct EpiGeluBwd {
  static constexpr int NB = 1;
  struct Aux {
    typename Elem<T>::raw_t a;
  };
  const T* A;
  T* dA;
  int64_t ld;
  int M, N;
  __device__ __forceinline__ void load(int m, int n, Aux& x) const {
    if (m < M && n < N) x.a = Elem<T>::load_once(A, (int64_t)m * ld + n, (int64_t)M * ld);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& x) const {
    if (m >= M || n >= N) return;
    const int64_t o = (int64_t)m * ld + n;
    float a[4], r[4];
    Elem<T>::unpack(x.a, a);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = v[0][j] * gelu_grad_f(a[j]);
    Elem<T>::store4(dA + o, r);
  }
};

// SwiGLU backward: acc = dH; dU = dH * SiLU(G); dG = dH * U * SiLU'(G),
// SiLU'(g) = s (1 + g (1 - s)), s = sigmoid(g).
template <class T>
struct EpiSwigluBwd {
  static constexpr int NB = 1;
  struct Aux {
    typename Elem<T>::raw_t g, u;
  };
  const T* G;
  const T* U;
  T* dG;
  T* dU;
  int64_t ld;
  int M, N;
  __device__ __forceinline__ void load(int m, int n, Aux& x) const {
    if (m < M && n < N) {
      const int64_t o = (int64_t)m * ld + n;
      x.g = Elem<T>::load_once(G, o, (int64_t)M * ld);
      x.u = Elem<T>::load_once(U, o, (int64_t)M * ld);
    }
  }
  __device__ __forceinline__ void operator()(int m, int n, const float (&v)[NB][4], const Aux& x) const {
    if (m >= M || n >= N) return;
    const int64_t o = (int64_t)m * ld + n;
    float g[4], u[4], dg[4], du[4];
    Elem<T>::unpack(x.g, g);
    Elem<T>::unpack(x.u, u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = sigmoid_f(g[j]);
      du[j] = v[0][j] * g[j] * s;
      dg[j] = v[0][j] * u[j] * s * (1.0f + g[j] * (1.0f - s));
    }
    Elem<T>::store4(dG + o, dg);
    Elem<T>::store4(dU + o, du);
  }
};

}  // namespace tp
