// attn_bwd_f32.hip - the fp32 backward of one SQuad pass (vector ALUs).
//
// The gradients of a softmax attention o_i = sum_j P_ij v_j with
// P_ij = softmax_j(scale <q_i, k_j>), given the upstream gradient dout, are
//   dv_j = sum_i P_ij dout_i,
//   dS_ij = P_ij (<dout_i, v_j> - D_i),   D_i = <dout_i, o_i> = sum_j P_ij <dout_i, v_j>,
//   dq_i = scale * sum_j dS_ij k_j,       dk_j = scale * sum_i dS_ij q_i.
// P is recomputed from the forward's row statistic lse_i (log2 domain, so
// P_ij = exp2(c <q_i, k_j> - lse_i), c = scale * log2 e).  The operator applies
// this to the global pass (values = the local output) and then to the local pass
// (upstream gradient = the local output's gradient); q and k collect both.
//
// Kind A: a workgroup of 256 threads runs 64 query rows of one unit (four lanes
// per row, a quarter of the dimensions each), streaming the unit's K and V rows
// through LDS in blocks of 32.  Kind B: the same with 64 key rows, streaming Q
// and dout rows (and lse, D) in blocks of 32 queries.
#include "squad_kernels.h"

namespace squad {
namespace {

constexpr int RB = 32;   // rows per LDS block
constexpr int PB = 64;   // own rows per workgroup

template <int D>
struct F32Cfg {
  static constexpr int DL = D / 4;      // dimensions per lane
  static constexpr int CPR = D / 4;     // 16-byte chunks per row
  static constexpr int PT = RB * CPR / 256;
  static_assert(RB * CPR % 256 == 0, "tiling");
};

// unit and row decode shared by both kinds (the chunks of a unit go to one XCD)
struct UnitPos {
  uint32_t u, s, b, h, chunk;
};
template <typename Args>
__device__ __forceinline__ bool unit_pos(const Args& a, UnitPos& p) {
  const uint32_t wg = blockIdx.x;
  const uint32_t jj = wg >> 3;
  p.chunk = jj % a.nchunks;
  p.u = (jj / a.nchunks) * 8 + (wg & 7);
  if (p.u >= a.units) return false;
  p.s = a.fBH.div(p.u);
  const uint32_t bh = p.u - p.s * a.BH;
  p.b = a.fHeads.div(bh);
  p.h = bh - p.b * a.heads;
  return true;
}

// sum over the four lanes of one row
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

template <int D, bool CUT, typename Args = BwdArgs>
__global__ __launch_bounds__(256) void bwd_dq_f32(Args a) {
  typedef F32Cfg<D> C;
  __shared__ __attribute__((aligned(16))) float ks[RB * D];
  __shared__ __attribute__((aligned(16))) float vs[RB * D];
  __shared__ uint32_t kmask;

  UnitPos p;
  if (!unit_pos(a, p)) return;
  // element offset of row r under map m (narrow maps: elements; wide: head rows)
  const uint32_t ru = a.row_unit > 1 ? a.row_unit : 1u;
  auto roff = [&](const auto& m, uint32_t r) -> uint64_t { return row_elems_rt(m.row_off(r), ru); };
  const uint32_t tid = threadIdx.x;
  const uint32_t L = a.L;
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, p.s);
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };
  const float* qg = (const float*)a.q + a.mqk.base(p.b, p.h, p.s);
  const float* kg = (const float*)a.k + a.mqk.base(p.b, p.h, p.s);
  const float* vg = (const float*)a.v + a.mv.base(p.b, p.h, p.s);
  const float* og = (const float*)a.o + a.mo.base(p.b, p.h, p.s);
  const float* dg = (const float*)a.dout + a.mdo.base(p.b, p.h, p.s);

  const uint32_t qi = p.chunk * PB + (tid >> 2);
  const uint32_t part = tid & 3;
  const bool qok = present(qi);
  float q[C::DL], dof[C::DL], dq[C::DL];
  float dsum = 0.f;
  {
    const float* qr = qg + (qok ? roff(a.mqk, qi) : 0) + part * C::DL;
    const float* dr = dg + (qok ? roff(a.mdo, qi) : 0) + part * C::DL;
    const float* orow = og + (qok ? roff(a.mo, qi) : 0) + part * C::DL;
#pragma unroll
    for (int i = 0; i < C::DL; ++i) {
      q[i] = qok ? qr[i] : 0.f;
      dof[i] = qok ? dr[i] : 0.f;
      dsum = fmaf(dof[i], qok ? orow[i] : 0.f, dsum);
      dq[i] = 0.f;
    }
  }
  dsum = quad_sum(dsum);
  const size_t row_id = (size_t)p.u * L + qi;
  const float lse = qok ? a.lse[row_id] : 0.f;
  if (qok && part == 0) a.dsum[row_id] = dsum;
  const float c = a.c;

  const uint32_t nkb = (L + RB - 1) / RB;
  for (uint32_t kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    if (tid < 64) {
      const uint64_t bits = __ballot(tid < RB && present(kb * RB + tid));
      if (tid == 0) kmask = (uint32_t)bits;
    }
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const uint32_t ch = tid + i * 256;
      const uint32_t r = ch / C::CPR, cc = ch % C::CPR;
      const uint32_t key = kb * RB + r;
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
#pragma unroll 4
    for (int j = 0; j < RB; ++j) {
      const float* kr = ks + j * D + part * C::DL;
      const float* vr = vs + j * D + part * C::DL;
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int i = 0; i < C::DL; ++i) {
        sd = fmaf(q[i], kr[i], sd);
        pd = fmaf(dof[i], vr[i], pd);
      }
      sd = quad_sum(sd);
      pd = quad_sum(pd);
      const float pij = ((km >> j) & 1) ? exp2f(fmaf(sd, c, -lse)) : 0.f;
      const float ds = pij * (pd - dsum);
#pragma unroll
      for (int i = 0; i < C::DL; ++i) dq[i] = fmaf(ds, kr[i], dq[i]);
    }
  }

  if (qok) {
    const uint64_t off = roff(a.mdq, qi) + part * C::DL;
    const int64_t base = a.mdq.base(p.b, p.h, p.s);
    float* acc = a.dq_acc + base + off;
#pragma unroll
    for (int i = 0; i < C::DL; i += 4) {
      float4 x = make_float4(dq[i] * a.scale, dq[i + 1] * a.scale, dq[i + 2] * a.scale, dq[i + 3] * a.scale);
      if (a.final_pass != kAccWrite) {
        const float4 y = *(const float4*)(acc + i);
        x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
      }
      *(float4*)((a.final_pass == kAccFinal ? (float*)a.dq + base + off : acc) + i) = x;
    }
  }
}

template <int D, bool CUT, typename Args = BwdArgs>
__global__ __launch_bounds__(256) void bwd_dkv_f32(Args a) {
  typedef F32Cfg<D> C;
  __shared__ __attribute__((aligned(16))) float qs[RB * D];
  __shared__ __attribute__((aligned(16))) float ds_[RB * D];
  __shared__ float lse_s[RB], dsum_s[RB];
  __shared__ uint32_t qmask;

  UnitPos p;
  if (!unit_pos(a, p)) return;
  // element offset of row r under map m (narrow maps: elements; wide: head rows)
  const uint32_t ru = a.row_unit > 1 ? a.row_unit : 1u;
  auto roff = [&](const auto& m, uint32_t r) -> uint64_t { return row_elems_rt(m.row_off(r), ru); };
  const uint32_t tid = threadIdx.x;
  const uint32_t L = a.L;
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, p.s);
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };
  const float* qg = (const float*)a.q + a.mqk.base(p.b, p.h, p.s);
  const float* kg = (const float*)a.k + a.mqk.base(p.b, p.h, p.s);
  const float* vg = (const float*)a.v + a.mv.base(p.b, p.h, p.s);
  const float* dg = (const float*)a.dout + a.mdo.base(p.b, p.h, p.s);

  const uint32_t kj = p.chunk * PB + (tid >> 2);   // this lane's key row
  const uint32_t part = tid & 3;
  const bool kok = present(kj);
  float k[C::DL], v[C::DL], dk[C::DL], dv[C::DL];
  {
    const float* kr = kg + (kok ? roff(a.mqk, kj) : 0) + part * C::DL;
    const float* vr = vg + (kok ? roff(a.mv, kj) : 0) + part * C::DL;
#pragma unroll
    for (int i = 0; i < C::DL; ++i) {
      k[i] = kok ? kr[i] : 0.f;
      v[i] = kok ? vr[i] : 0.f;
      dk[i] = 0.f;
      dv[i] = 0.f;
    }
  }
  const float c = a.c;
  const size_t unit_rows = (size_t)p.u * L;

  const uint32_t nqb = (L + RB - 1) / RB;
  for (uint32_t qb = 0; qb < nqb; ++qb) {
    __syncthreads();
    if (tid < 64) {
      const uint32_t r = qb * RB + tid;
      const bool ok = tid < RB && present(r);
      const uint64_t bits = __ballot(ok);
      if (tid == 0) qmask = (uint32_t)bits;
      if (tid < RB) {
        lse_s[tid] = ok ? a.lse[unit_rows + r] : 0.f;
        dsum_s[tid] = ok ? a.dsum[unit_rows + r] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const uint32_t ch = tid + i * 256;
      const uint32_t r = ch / C::CPR, cc = ch % C::CPR;
      const uint32_t qr = qb * RB + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (present(qr)) {
        x = *(const float4*)(qg + roff(a.mqk, qr) + cc * 4);
        y = *(const float4*)(dg + roff(a.mdo, qr) + cc * 4);
      }
      *(float4*)(qs + r * D + cc * 4) = x;
      *(float4*)(ds_ + r * D + cc * 4) = y;
    }
    __syncthreads();
    const uint32_t qm = qmask;
#pragma unroll 4
    for (int i = 0; i < RB; ++i) {
      const float* qr = qs + i * D + part * C::DL;
      const float* dr = ds_ + i * D + part * C::DL;
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < C::DL; ++e) {
        sd = fmaf(qr[e], k[e], sd);
        pd = fmaf(dr[e], v[e], pd);
      }
      sd = quad_sum(sd);
      pd = quad_sum(pd);
      const float pij = ((qm >> i) & 1) ? exp2f(fmaf(sd, c, -lse_s[i])) : 0.f;
      const float dsv = pij * (pd - dsum_s[i]);
#pragma unroll
      for (int e = 0; e < C::DL; ++e) {
        dv[e] = fmaf(pij, dr[e], dv[e]);
        dk[e] = fmaf(dsv, qr[e], dk[e]);
      }
    }
  }

  if (kok) {
    const int64_t kbase = a.mdk.base(p.b, p.h, p.s);
    const uint64_t koff = roff(a.mdk, kj) + part * C::DL;
    float* acc = a.dk_acc + kbase + koff;
    float* vrow = (float*)a.dv + a.mdv.base(p.b, p.h, p.s) + roff(a.mdv, kj) + part * C::DL;
#pragma unroll
    for (int e = 0; e < C::DL; e += 4) {
      float4 x = make_float4(dk[e] * a.scale, dk[e + 1] * a.scale, dk[e + 2] * a.scale, dk[e + 3] * a.scale);
      if (a.final_pass != kAccWrite) {
        const float4 y = *(const float4*)(acc + e);
        x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
      }
      *(float4*)((a.final_pass == kAccFinal ? (float*)a.dk + kbase + koff : acc) + e) = x;
      *(float4*)(vrow + e) = make_float4(dv[e], dv[e + 1], dv[e + 2], dv[e + 3]);
    }
  }
}

template <int D, typename Args>
hipError_t launch(const Args& a, bool kind_b, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)((a.units + 7) / 8) * 8 * a.nchunks;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 grid((uint32_t)blocks), block(256);
  if constexpr (std::is_same<Args, BwdArgs>::value) {
    if (a.cut.on) {
      if (kind_b) hipLaunchKernelGGL((bwd_dkv_f32<D, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((bwd_dq_f32<D, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  } else if (a.cut.on) {
    return hipErrorInvalidValue;
  }
  if (kind_b) hipLaunchKernelGGL((bwd_dkv_f32<D, false, Args>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((bwd_dq_f32<D, false, Args>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(BwdArgs a, int head_dim, bool kind_b, hipStream_t stream) {
  a.nchunks = (a.L + PB - 1) / PB;
  if (head_dim == 128) return launch<128>(a, kind_b, stream);
  if (head_dim == 64) return launch<64>(a, kind_b, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32_k(BwdArgsK a, int head_dim, bool kind_b, hipStream_t stream) {
  a.nchunks = (a.L + PB - 1) / PB;
  if (head_dim == 128) return launch<128>(a, kind_b, stream);
  if (head_dim == 64) return launch<64>(a, kind_b, stream);
  return hipErrorInvalidValue;
}

}  // namespace squad
