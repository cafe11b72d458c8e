// Shared device types and helpers for the gfx950 kernels of libtpshard.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// ---- kernel launches -------------------------------------------------------
// Every kernel of the library is launched through tp_launch.  While a
// profiling scope is open on the calling thread (tp_profile_arm), the launch
// carries the scope's events: the start event on the scope's first kernel
// and the stop event on each kernel, so that they hold the first kernel's
// start and the last one's end as the dispatches themselves timestamp them
// (no marker packets between kernels).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool started = false;
};
inline thread_local LaunchEvents* g_launch_events = nullptr;

template <typename F, typename... Args>
inline void tp_launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream, Args... args) {
  if (LaunchEvents* ev = g_launch_events) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev->started ? nullptr : ev->start, ev->stop, 0u,
                          args...);
    ev->started = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- buffer loads ----------------------------------------------------------
// Raw buffer loads through a buffer resource descriptor: the hardware returns
// zeros for any byte offset at or beyond the descriptor's size, so ragged
// tile edges are handled by pointing invalid lanes at kOOB instead of
// branching around the load.  Operands handed to these loads are < 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  // dword 3 = 0x00020000: 32-bit data format, the raw-buffer setting on gfx9 parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// bf16 is carried as its raw 16 bits (uint16_t) in memory.
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats -> packed bf16 pair (lo in bits 0-15), round-to-nearest-even, in
// one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Storage policies: load/store 4 consecutive elements as float.  Results are
// stored non-temporally and the epilogues' saved tensors, read once, are
// loaded with the sc1 cache policy (together 4% on the SwiGLU-backward GEMM
// on gfx950).
template <class T> struct Elem;
template <> struct Elem<uint16_t> {
  typedef u32x2 raw_t;  // 4 elements as loaded, unpacked later
  __device__ __forceinline__ static raw_t load_raw(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
  // elements o .. o+3 of a tensor of `extent` elements (< 2^31 bytes) at `base`
  __device__ __forceinline__ static raw_t load_once(const uint16_t* base, int64_t o, int64_t extent) {
    return __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(base, (uint32_t)(extent * 2)), (uint32_t)(o * 2), 0,
                                                2 /* sc1 */);
  }
  __device__ __forceinline__ static void unpack(const raw_t& w, float (&v)[4]) {
    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
  }
  __device__ __forceinline__ static void load4(const uint16_t* p, float (&v)[4]) {
    u32x2 w = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
  }
  __device__ __forceinline__ static void store4(uint16_t* p, const float (&v)[4]) {
    u32x2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
};
template <> struct Elem<float> {
  typedef f32x4 raw_t;
  __device__ __forceinline__ static raw_t load_raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ static raw_t load_once(const float* base, int64_t o, int64_t) {
    return *reinterpret_cast<const f32x4*>(base + o);
  }
  __device__ __forceinline__ static void unpack(const raw_t& w, float (&v)[4]) {
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  __device__ __forceinline__ static void load4(const float* p, float (&v)[4]) {
    f32x4 w = *reinterpret_cast<const f32x4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  __device__ __forceinline__ static void store4(float* p, const float (&v)[4]) {
    f32x4 w = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
};

// SplitMix64 output number n (1-based) of the stream seeded with `seed`
// (Steele, Lea & Flood, OOPSLA 2014; constants of the published reference
// implementation).
__device__ __forceinline__ uint64_t splitmix64_nth(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Dropout decision for flat element index idx of the [rows, cols] output:
// keep iff the high 32 bits of output idx+1 are >= thr = floor(p * 2^32).
__device__ __forceinline__ bool dropout_keep(uint64_t seed, uint64_t idx, uint32_t thr) {
  return (uint32_t)(splitmix64_nth(seed, idx + 1) >> 32) >= thr;
}

// ---- activations (fp32) ----------------------------------------------------
// GeLU in its exact erf form x * Phi(x); SiLU(x) = x * sigmoid(x).
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad_f(float x) {
  // Phi(x) + x * phi(x)
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * __expf(-0.5f * x * x);
}
// v_rcp_f32 (about 1 ulp) instead of an IEEE division
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

}  // namespace tp
