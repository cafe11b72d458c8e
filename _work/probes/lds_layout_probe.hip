// Counter probe of the library's 256x256 GEMM tile: three rounds of two single
// launches, one with both operands K-contiguous (8192 x 3584 x 8192, the MLP
// dH shape) and one with both M/N-contiguous (3584 x 8192 x 8192, the dW2
// shape), on synthetic bf16 data, so that rocprofv3 counters can be read per
// operand layout.  Not part of the library; built by hand:
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -I include attention_column_gemm_amd/probes/lds_layout_probe.hip -o lds_layout_probe
#include <cstdio>
#include <cstdlib>
#include "../csrc/gemm_dma.hpp"
#include "../csrc/epilogues.hpp"
using namespace tp;
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1);} } while (0)

__global__ void fill(uint16_t* p, size_t n, uint32_t seed) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint32_t x = (uint32_t)i * 2654435761u ^ seed; x ^= x >> 13; x *= 0x5bd1e995u; x ^= x >> 15;
    const float f = ((x & 0xffff) / 32768.0f - 1.0f);
    p[i] = (uint16_t)(__float_as_uint(f) >> 16);
  }
}

int main() {
  const size_t n = (size_t)8192 * 8192;
  uint16_t *A, *B; float* C;
  CK(hipMalloc(&A, n * 2)); CK(hipMalloc(&B, n * 2)); CK(hipMalloc(&C, n * 4));
  fill<<<4096, 256>>>(A, n, 1); fill<<<4096, 256>>>(B, n, 2);
  CK(hipDeviceSynchronize());
  // dH-like: M=8192, N=3584, K=8192, A [M,K], B [N,K]
  GemmProblem kk{}; kk.M = 8192; kk.N = 3584; kk.nseg = 1; kk.K[0] = 8192;
  kk.A[0] = kk.A[1] = A; kk.B[0][0] = kk.B[1][0] = kk.B[0][1] = kk.B[1][1] = B;
  kk.lda[0] = kk.lda[1] = 8192; kk.ldb[0] = kk.ldb[1] = 8192;
  // dW2-like: M=3584, N=8192, K=8192, A [K,M], B [K,N]
  GemmProblem mm{}; mm.M = 3584; mm.N = 8192; mm.nseg = 1; mm.K[0] = 8192;
  mm.A[0] = mm.A[1] = A; mm.B[0][0] = mm.B[1][0] = mm.B[0][1] = mm.B[1][1] = B;
  mm.lda[0] = mm.lda[1] = 3584; mm.ldb[0] = mm.ldb[1] = 8192;
  for (int r = 0; r < 3; ++r) {
    EpiStore<float> e1{C, kk.N, kk.M, kk.N};
    CK((launch_gemm_dma<256, 256, 4, 2, 64, KMAJOR, KMAJOR>(kk, e1, 0)));
    EpiStore<float> e2{C, mm.N, mm.M, mm.N};
    CK((launch_gemm_dma<256, 256, 4, 2, 64, MNMAJOR, MNMAJOR>(mm, e2, 0)));
  }
  CK(hipDeviceSynchronize());
  printf("done\n");
  return 0;
}
