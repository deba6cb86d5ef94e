// permute.hip - exact row-permutation copies: the window gather and scatter and the
// window-to-group regroup (the tensor reshaping the method is built from; technical
// summary, "Belangrijkste Bijdragen").
//
// Each thread moves 16-byte chunks; the row index is taken in the contiguous
// side's order, so consecutive lanes write (gather, regroup) or read (scatter)
// consecutive bytes, and the permuted side is touched in whole rows of
// head_dim * elem_bytes (256 B for bf16 at head_dim 128).
#include "squad_kernels.h"

namespace squad {
namespace {

constexpr int CPT = 4;  // chunks per thread

__global__ __launch_bounds__(256) void row_copy_kernel(CopyArgs a) {
  const uint64_t total = (uint64_t)a.rows << a.row_chunks_log2;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const uint64_t c = (uint64_t)blockIdx.x * (256 * CPT) + i * 256 + threadIdx.x;
    if (c >= total) return;
    const uint32_t e = (uint32_t)(c >> a.row_chunks_log2);
    const uint32_t cc = (uint32_t)c & ((1u << a.row_chunks_log2) - 1);
    const uint32_t t = a.fL.div(e);
    const uint32_t r = e - t * a.L;
    const uint32_t bh = a.fU.div(t);
    const uint32_t s = t - bh * a.U;
    const uint32_t b = a.fHeads.div(bh);
    const uint32_t h = bh - b * a.heads;
    const uint32_t ru = a.row_unit > 1 ? a.row_unit : 1u;
    const int64_t so = a.ms.base(b, h, s) + (int64_t)row_elems_rt(a.ms.row_off(r), ru);
    const int64_t dso = a.md.base(b, h, s) + (int64_t)row_elems_rt(a.md.row_off(r), ru);
    const uint4 x = *(const uint4*)((const char*)a.src + (so * a.elem_bytes) + (uint64_t)cc * 16);
    *(uint4*)((char*)a.dst + (dso * a.elem_bytes) + (uint64_t)cc * 16) = x;
  }
}

}  // namespace

hipError_t launch_row_copy(CopyArgs a, hipStream_t stream) {
  const uint64_t total = (uint64_t)a.rows << a.row_chunks_log2;
  const uint64_t blocks = (total + 256 * CPT - 1) / (256 * CPT);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(row_copy_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace squad
