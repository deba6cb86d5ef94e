// attn_f32.hip - the fp32 attention engine behind both SQuad passes.
//
// Same contract as the bf16 engine (one softmax attention per unit of L rows; the
// standard softmax of both passes, technical summary "1. SQuad-Attention
// Operator"), kept entirely in fp32 on the vector ALUs: no operand is rounded to a
// narrower type.  A workgroup of 256 threads runs 64 query rows of one unit; four
// neighbouring lanes share one query, each holding a quarter of its dimensions, and
// combine their partial dot products with two butterfly exchanges.  Keys and values
// stream through LDS in blocks of 32 rows with an online softmax.
#include "squad_kernels.h"

namespace squad {
namespace {

constexpr int KB = 32;   // keys per LDS block
constexpr int QPB = 64;  // queries per workgroup

// CUT: the grid is not a whole number of tiles; absent rows are neither keys nor
// stored queries.
template <int D, bool CUT, typename Args = AttnArgs>
__global__ __launch_bounds__(256) void attn_f32_kernel(Args a) {
  constexpr int DL = D / 4;        // dimensions per lane
  constexpr int CPR = D / 4;       // 16-byte chunks per row (4 floats each)
  constexpr int CH = KB * CPR;     // chunks per K (or V) block
  constexpr int PT = CH / 256;     // chunks per thread
  static_assert(CH % 256 == 0, "tiling");

  __shared__ __attribute__((aligned(16))) float ks[KB * D];
  __shared__ __attribute__((aligned(16))) float vs[KB * D];
  __shared__ uint32_t kmask;   // present keys of the current block

  const uint32_t tid = threadIdx.x;
  const uint32_t wg = blockIdx.x;
  const uint32_t xcd = wg & 7;
  const uint32_t jj = wg >> 3;
  const uint32_t chunk = jj % a.nchunks;
  const uint32_t u = (jj / a.nchunks) * 8 + xcd;
  if (u >= a.units) return;

  const uint32_t s = a.fBH.div(u);
  const uint32_t bh = u - s * a.BH;
  const uint32_t b = a.fHeads.div(bh);
  const uint32_t h = bh - b * a.heads;
  const float* qg = (const float*)a.q + a.mqk.base(b, h, s);
  const float* kg = (const float*)a.k + a.mqk.base(b, h, s);
  const float* vg = (const float*)a.v + a.mv.base(b, h, s);
  float* og = (float*)a.o + a.mo.base(b, h, s);

  const uint32_t L = a.L;
  // element offset of row r under map m (narrow maps: elements; wide: head rows)
  const uint32_t ru = a.row_unit > 1 ? a.row_unit : 1u;
  auto roff = [&](const auto& m, uint32_t r) -> uint64_t { return row_elems_rt(m.row_off(r), ru); };
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, s);
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };
  const uint32_t qi = chunk * QPB + (tid >> 2);   // this lane's query row
  const uint32_t part = tid & 3;                  // which quarter of the dimensions
  const bool qok = present(qi);

  float q[DL], acc[DL];
  {
    const float* qr = qg + (qok ? roff(a.mqk, qi) : 0) + part * DL;
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      q[i] = qok ? qr[i] : 0.f;
      acc[i] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.c;

  const uint32_t nkb = (L + KB - 1) / KB;
  for (uint32_t kb = 0; kb < nkb; ++kb) {
    __syncthreads();   // previous block fully consumed
    if (tid < 64) {
      const uint64_t bits = __ballot(tid < KB && present(kb * KB + tid));
      if (tid == 0) kmask = (uint32_t)bits;
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const uint32_t ch = tid + i * 256;
      const uint32_t r = ch / CPR, cc = ch % CPR;
      const uint32_t key = kb * KB + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (present(key)) {
        kv = *(const float4*)(kg + roff(a.mqk, key) + cc * 4);
        vv = *(const float4*)(vg + roff(a.mv, key) + cc * 4);
      }
      *(float4*)(ks + r * D + cc * 4) = kv;
      *(float4*)(vs + r * D + cc * 4) = vv;
    }
    __syncthreads();
    const uint32_t km = kmask;

    float sc[KB];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float* kr = ks + j * D + part * DL;
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < DL; ++i) d0 = fmaf(q[i], kr[i], d0);
      d0 += __shfl_xor(d0, 1, 64);
      d0 += __shfl_xor(d0, 2, 64);
      sc[j] = ((km >> j) & 1) ? d0 * c : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      sc[j] = exp2f(sc[j] - m_new);
      ps += sc[j];
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float* vr = vs + j * D + part * DL;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] = fmaf(sc[j], vr[i], acc[i]);
    }
  }

  if (qok) {
    if (a.lse && part == 0) a.lse[(size_t)u * L + qi] = m_run + __log2f(l_run);
    const float inv = 1.f / l_run;
    float* orow = og + roff(a.mo, qi) + part * DL;
#pragma unroll
    for (int i = 0; i < DL; i += 4)
      *(float4*)(orow + i) = make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
  }
}

template <int D, typename Args>
hipError_t launch(const Args& a, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)((a.units + 7) / 8) * 8 * a.nchunks;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if constexpr (std::is_same<Args, AttnArgs>::value) {
    if (a.cut.on) {
      hipLaunchKernelGGL((attn_f32_kernel<D, true>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
  } else if (a.cut.on) {
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((attn_f32_kernel<D, false, Args>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(AttnArgs a, int head_dim, hipStream_t stream) {
  a.nchunks = (a.L + QPB - 1) / QPB;
  if (head_dim == 128) return launch<128>(a, stream);
  if (head_dim == 64) return launch<64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32_k(AttnArgsK a, int head_dim, hipStream_t stream) {
  a.nchunks = (a.L + QPB - 1) / QPB;
  if (head_dim == 128) return launch<128>(a, stream);
  if (head_dim == 64) return launch<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace squad
