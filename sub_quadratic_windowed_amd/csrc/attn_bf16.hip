// attn_bf16.hip - the bf16 attention engine behind both SQuad passes (gfx950 MFMA).
//
// One workgroup runs one query chunk (32 rows per wave) of one unit (a window in
// the local pass, an offset group in the global pass) against all of the unit's
// keys, streamed through LDS in blocks of 64 keys with an online softmax.  The
// standard softmax of both passes (technical summary, "1. SQuad-Attention
// Operator") is computed exactly: row max, exp2 of the shifted logits, row sum and
// a final division, in fp32.
//
// Products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   S^T = K * Q^T   (A = 32 keys x 16 dims from LDS, B = Q^T from registers)
//   O^T = V^T * P^T (A = V^T read with ds_read_b64_tr_b16, B = P^T from registers)
// Computing the transposes puts one query per lane (lane % 32), so the softmax row
// statistics are per-lane scalars; only the two 32-lane halves of the wave meet, in
// one cross-half exchange per key block.  The C/D layout of the 32x32 MFMA gives lane
// l, register r the element (row 8*(r/4) + 4*(l/32) + r%4, column l%32); P^T leaves the
// S^T registers in exactly the k-slot order the second MFMA needs when V^T is read
// with the matching key permutation, so P never moves between lanes.
#include "squad_kernels.h"

namespace squad {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int BN = 64;  // keys per LDS block

// 16-bit value types of the weights-times-values product: bf16 for bf16 values, fp16
// for the fp16 local output the global pass reads (see squad_api.hip).
template <typename T> struct Vec;
template <> struct Vec<__bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Vec<_Float16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ int64_t shfl64(int64_t x, int src) {
  int lo = __shfl((int)(uint32_t)(uint64_t)x, src, 64);
  int hi = __shfl((int)(uint32_t)((uint64_t)x >> 32), src, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32, 64); }

// VT: type of v (and of the attention weights in the second product); OT: type of out.
template <int D, int NW, typename VT, typename OT>
__global__ __launch_bounds__(64 * NW) void attn_bf16_kernel(AttnArgs a) {
  typedef typename Vec<VT>::x8 vx8;
  typedef typename Vec<VT>::x4 vx4;
  typedef typename Vec<OT>::x4 ox4;
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;
  constexpr int KP = D + 8;             // LDS row pitch in elements (272 B for D = 128)
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int KV = BN * KP;           // elements of one K or V buffer
  constexpr int LDS = (4 * KV > BM * KP) ? 4 * KV : BM * KP;
  constexpr int RPI = NT / CPR;         // rows one pass of the workgroup covers
  constexpr int KVI = BN / RPI;         // 16-byte chunks per thread per K (or V) block
  constexpr int WR = 64 / CPR;          // rows one wave covers per pass
  constexpr int QI = 32 / WR;           // passes for a wave's 32 rows
  static_assert(BN % RPI == 0 && 32 % WR == 0, "tiling");

  __shared__ __attribute__((aligned(16))) __bf16 smem[LDS];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t half = lane >> 5;
  const uint32_t l32 = lane & 31;

  // workgroup -> (unit, query chunk); the chunks of one unit go to one XCD
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

  const __bf16* qg = (const __bf16*)a.q + a.mqk.base(b, h, s);
  const __bf16* kg = (const __bf16*)a.k + a.mqk.base(b, h, s);
  const VT* vg = (const VT*)a.v + a.mv.base(b, h, s);
  OT* og = (OT*)a.o + a.mo.base(b, h, s);

  const uint32_t L = a.L;
  const uint32_t nkb = (L + BN - 1) / BN;
  const uint32_t q0 = chunk * BM + wave * 32;   // first query row of this wave
  const bool active = q0 < L;

  const uint32_t ccol = tid % CPR;              // chunk column for K/V staging
  const uint32_t crow = tid / CPR;              // row within a staging pass
  const uint32_t wcol = lane % CPR;             // chunk column for per-wave Q/O passes
  const uint32_t wrow = lane / CPR;

  // ---- K/V block prefetch into registers
  uint4 kreg[KVI], vreg[KVI];
  auto prefetch = [&](uint32_t kb) {
    const uint32_t key = kb * BN + lane;        // lane l locates key row l of the block
    const bool ok = key < L;
    const int64_t ok_k = ok ? a.mqk.row_off(key) : -1;
    const int64_t ok_v = ok ? a.mv.row_off(key) : -1;
#pragma unroll
    for (int i = 0; i < KVI; ++i) {
      const int r = crow + i * RPI;
      const int64_t ok_ = shfl64(ok_k, r);
      const int64_t ov_ = shfl64(ok_v, r);
      uint4 zk = make_uint4(0, 0, 0, 0), zv = zk;
      if (ok_ >= 0) zk = *(const uint4*)(kg + ok_ + ccol * 8);
      if (ov_ >= 0) zv = *(const uint4*)(vg + ov_ + ccol * 8);
      kreg[i] = zk;
      vreg[i] = zv;
    }
  };
  auto stage = [&](int buf) {
    __bf16* ks = smem + buf * KV;
    __bf16* vs = smem + (2 + buf) * KV;
#pragma unroll
    for (int i = 0; i < KVI; ++i) {
      const int r = crow + i * RPI;
      *(uint4*)(ks + r * KP + ccol * 8) = kreg[i];
      *(uint4*)(vs + r * KP + ccol * 8) = vreg[i];
    }
  };

  // ---- prologue: Q rows of this wave through LDS into MFMA B-operand registers
  const uint32_t qrow_l = q0 + l32;
  const int64_t qoff_l = (qrow_l < L) ? a.mqk.row_off(qrow_l) : -1;
  uint4 qreg[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int64_t o = shfl64(qoff_l, wrow + i * WR);
    qreg[i] = make_uint4(0, 0, 0, 0);
    if (o >= 0) qreg[i] = *(const uint4*)(qg + o + wcol * 8);
  }
  prefetch(0);
  {
    __bf16* qs = smem + wave * 32 * KP;
#pragma unroll
    for (int i = 0; i < QI; ++i) *(uint4*)(qs + (wrow + i * WR) * KP + wcol * 8) = qreg[i];
  }
  __syncthreads();
  bf16x8 qf[D / 16];
  {
    const __bf16* qs = smem + wave * 32 * KP + l32 * KP + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qs + kk * 16);
  }
  __syncthreads();
  stage(0);
  __syncthreads();

  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
  float m_run = -INFINITY;   // running max of scaled logits (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum
  const float c = a.c;

  for (uint32_t kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool has_next = kb + 1 < nkb;
    if (has_next) prefetch(kb + 1);

    if (active) {
      const __bf16* ks = smem + buf * KV;
      const __bf16* vs = smem + (2 + buf) * KV;
      // S^T tiles: keys 0-31 and 32-63 of the block against this wave's 32 queries
      f32x16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 k0 = *(const bf16x8*)(ks + l32 * KP + kk * 16 + half * 8);
        const bf16x8 k1 = *(const bf16x8*)(ks + (32 + l32) * KP + kk * 16 + half * 8);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], s1, 0, 0, 0);
      }
      // keys past the end of the unit take no weight
      if ((kb + 1) * BN > L) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t kr = kb * BN + 8 * (r / 4) + 4 * half + (r % 4);
          if (kr >= L) s0[r] = -INFINITY;
          if (kr + 32 >= L) s1[r] = -INFINITY;
        }
      }
      float mx = s0[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
      mx = fmaxf(mx, xhalf(mx));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float ps = 0.f;
      vx8 pb[4];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -m_new));
        ps += p0 + p1;
        pb[r / 8][r % 8] = (VT)p0;
        pb[2 + r / 8][r % 8] = (VT)p1;
      }
      l_run = l_run * alpha + ps;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha;
      // O^T += V^T P^T, 16 keys per MFMA
      const uint32_t trow = 4 * half + ((lane & 15) >> 2);
      const uint32_t tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int jk = 0; jk < 4; ++jk) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          const __bf16* p1 = vs + (16 * jk + trow) * KP + mt * 32 + tcol;
          const __bf16* p2 = p1 + 8 * KP;
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(__attribute__((address_space(3))) __bf16*)p1);
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(__attribute__((address_space(3))) __bf16*)p2);
          vx8 va;
          const vx4 lo4 = __builtin_bit_cast(vx4, lo);
          const vx4 hi4 = __builtin_bit_cast(vx4, hi);
          va[0] = lo4[0]; va[1] = lo4[1]; va[2] = lo4[2]; va[3] = lo4[3];
          va[4] = hi4[0]; va[5] = hi4[1]; va[6] = hi4[2]; va[7] = hi4[3];
          acc[mt] = Vec<VT>::mfma(va, pb[jk], acc[mt]);
        }
      }
    }
    if (has_next) stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, stage rows in LDS, store 16-byte chunks
  const float inv = 1.f / (l_run + xhalf(l_run));
  if (active) {
    __bf16* os = smem + wave * 32 * KP + l32 * KP;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ox4 w;
        w[0] = (OT)(acc[mt][4 * g + 0] * inv);
        w[1] = (OT)(acc[mt][4 * g + 1] * inv);
        w[2] = (OT)(acc[mt][4 * g + 2] * inv);
        w[3] = (OT)(acc[mt][4 * g + 3] * inv);
        *(ox4*)(os + mt * 32 + 8 * g + 4 * half) = w;
      }
  }
  __syncthreads();
  if (active) {
    const int64_t ooff_l = (qrow_l < L) ? a.mo.row_off(qrow_l) : -1;
    const __bf16* os = smem + wave * 32 * KP;
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int r = wrow + i * WR;
      const int64_t o = shfl64(ooff_l, r);
      if (o >= 0) *(uint4*)(og + o + wcol * 8) = *(const uint4*)(os + r * KP + wcol * 8);
    }
  }
}

template <int D, int NW, typename VT, typename OT>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const uint32_t groups = (a.units + 7) / 8;
  const uint64_t blocks = (uint64_t)groups * 8 * a.nchunks;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, VT, OT>), dim3((uint32_t)blocks), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

template <int D, typename VT, typename OT>
hipError_t launch_nw(const AttnArgs& a, int nw, hipStream_t stream) {
  return nw == 4 ? launch<D, 4, VT, OT>(a, stream) : launch<D, 2, VT, OT>(a, stream);
}

template <typename VT, typename OT>
hipError_t launch_types(const AttnArgs& a, int head_dim, int nw, hipStream_t stream) {
  if (head_dim == 128) return launch_nw<128, VT, OT>(a, nw, stream);
  if (head_dim == 64) return launch_nw<64, VT, OT>(a, nw, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// Waves per workgroup: 2 for units of at most 64 rows, else 4 (two 4-wave
// workgroups fit one CU's registers and LDS).
hipError_t launch_attn_bf16(AttnArgs a, int head_dim, VType vtype, hipStream_t stream) {
  const uint32_t tiles = (a.L + 31) / 32;
  const int nw = tiles > 2 ? 4 : 2;
  a.nchunks = (tiles + nw - 1) / nw;
  switch (vtype) {
    case VType::kBf16ToBf16: return launch_types<__bf16, __bf16>(a, head_dim, nw, stream);
    case VType::kBf16ToF16: return launch_types<__bf16, _Float16>(a, head_dim, nw, stream);
    case VType::kF16ToBf16: return launch_types<_Float16, __bf16>(a, head_dim, nw, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace squad
