// LDS-direct loads and explicit wait/barrier helpers shared by the kernels
// that stage HBM tiles straight into LDS (the GEMM and the attention
// backward).
#pragma once

#include "common.hpp"

namespace tp {
namespace lds {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor in four SGPRs (base, stride 0, size, raw dword format).
__device__ __forceinline__ u32x4 sgpr_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, num_bytes, 0x00020000u};
}

// One 16-byte load per lane from `rsrc` at byte offset `voff` into LDS at
// m0 + 16 * lane.  Written in assembly so that the compiler neither inserts
// conservative waits for it nor reorders LDS accesses across it; completion
// is tracked explicitly with wait_vmcnt.  Offsets at or past the descriptor's
// size read zeros.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rsrc)
               : "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// ds_read_b64_tr_b16 from LDS byte address `off`: within each 16-lane group,
// lane R names row (R / 4) of four consecutive k rows and the four 16-bit
// elements at column 4 * (R % 4) of a 16-wide column run; lane i then receives
// the four k rows' elements of column i.
__device__ __forceinline__ v4i16 read_tr16(const lds_u8* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_u8*>(base) + off));
}

}  // namespace lds
}  // namespace tp
