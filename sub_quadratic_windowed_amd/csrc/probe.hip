// probe.hip - a measuring kernel: the sustained bf16 MFMA rate of this card.
//
// Every wave runs independent chains of v_mfma_f32_32x32x16_bf16 on operands
// drawn from a per-lane hash (random-looking data: the rate with constant
// operands is higher, because the matrix cores draw less power).  Nothing but the
// products runs in the loop, so the measured rate is the ceiling a kernel that
// also loads, reduces and stores can approach on the same card and clock.
#include "squad_kernels.h"

namespace squad {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 4;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // a 32-bit integer hash (xorshift-multiply), only to spread operand bits
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int32_t iters, uint32_t seed) {
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[CHAINS], b[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // values in [-1, 1): the bf16 of a uniform draw from the hash
      const uint32_t h = mix32(gid * 64u + (uint32_t)(j * 8 + e) + seed);
      a[j][e] = (__bf16)((float)(h & 0xffffu) / 32768.f - 1.f);
      b[j][e] = (__bf16)((float)(h >> 16) / 32768.f - 1.f);
    }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  // rounds of four, so every operand index is static
  for (int32_t it = 0; it < iters; it += 4) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int j = 0; j < CHAINS; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + r4) & (CHAINS - 1)], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[gid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int32_t blocks, int32_t iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, out, iters, 12345u);
  return hipGetLastError();
}

}  // namespace squad
