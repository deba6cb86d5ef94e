// attn_bwd_bf16.hip - the 16-bit backward of one SQuad pass (gfx950 MFMA).
//
// Gradients of the unit attentions o_i = sum_j P_ij v_j (P_ij = softmax_j of the
// scaled logits), given the upstream gradient dout:
//   dv_j = sum_i P_ij dout_i,    dS_ij = P_ij (<dout_i, v_j> - D_i),  D_i = <dout_i, o_i>,
//   dq_i = scale * sum_j dS_ij k_j,   dk_j = scale * sum_i dS_ij q_i,
// with P recomputed as exp2(c <q_i, k_j> - lse_i) from the forward's row statistic.
//
// Kind A (one query chunk of 32 rows per wave): Q^T and dout^T stay in registers as
// B operands; per block of 32 keys
//   S^T  = K * Q^T       (A = K rows from LDS)
//   dP^T = V * dout^T    (A = V rows from LDS)
//   dq^T += K^T * dS^T   (A = K^T from LDS with the transposing read, B = dS^T in
//                         registers: the S^T output layout is the B layout once
//                         K^T is read with the matching key permutation)
// so each lane owns one query and its statistics (lse, D) are per-lane scalars.
// Kind B (one key chunk of 32 rows per wave): K^T in registers, the workgroup's own
// V rows in LDS (read as B operands; as registers they would leave no room for
// the two accumulators); per block of 32 queries
//   S  = Q * K^T,  dP = dout * V^T   (A = Q and dout rows from LDS)
//   dv^T += dout^T * P,  dk^T += Q^T * dS   (A = transposing reads of dout and Q)
// each lane owning one key; the block's 32 lse and D values arrive in LDS by one
// more direct load.
//
// LDS blocks hold 32 rows of 16-bit elements as 8 groups of 4 rows; in group g the
// 16-byte chunk c of row r sits at slot 4 * (c ^ (g % 4)) + r % 4.  Row reads (A
// operands, 16 bytes per lane) and transposing reads (ds_read_b64_tr_b16) are
// then both free of bank conflicts, and a block is filled by direct global -> LDS
// loads (one 16-byte chunk per lane).  Kind A keeps three stages and requests each
// block two steps ahead; kind B (whose own V rows take the room of a third stage)
// keeps two and requests the next block before using the current one.  Units of
// at most 512 rows form their rows' byte offsets once, into LDS tables.
//
// Units of at most 64 rows (whole tilings) take one fused kernel instead: a
// two-wave workgroup holds the whole unit, forms S and dP once (kind B's layout)
// and passes dS through LDS to the dq product (see bwd_small_bf16).
//
// Products are bf16 with fp32 accumulation, except the global pass's dP^T: its
// values are the fp16 local output, so it runs on fp16 MFMAs against dout scaled
// per row by a power of two into fp16 range (undone on the fp32 result).  Elsewhere
// fp16 operands are converted to bf16 on the way in.  dS and P are rounded to bf16
// for their products.
#include "squad_kernels.h"

namespace squad {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BN = 32;   // rows per streamed block

// NW waves per workgroup (4, or 2 for units of at most 64 rows), 32 own rows each
template <int D, int NW>
struct BCfg {
  static constexpr int BM = 32 * NW;             // own rows per workgroup
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int GRP = 4 * D;             // elements of one 4-row group
  static constexpr int GPI = 64 / (4 * CPR);    // groups filled by one direct load
  static constexpr int VINS = BN * CPR / 64;    // direct loads per block
  static constexpr int VPW = VINS / NW;         // ... per wave
  static_assert(VPW * NW == VINS && VPW >= 1, "loads split evenly over the waves");
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 to_bf16(f16x8 x) {
  bf16x8 y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (__bf16)(float)x[i];
  return y;
}

// 8 consecutive 16-bit elements as a bf16 fragment (fp16 storage converted)
template <bool F16>
__device__ __forceinline__ bf16x8 frag(uint4 raw) {
  if constexpr (F16) return to_bf16(__builtin_bit_cast(f16x8, raw));
  else return __builtin_bit_cast(bf16x8, raw);
}

template <bool F16>
__device__ __forceinline__ float elem(const void* p, int i) {
  if constexpr (F16) return (float)((const _Float16*)p)[i];
  else return (float)((const __bf16*)p)[i];
}

// the lane's half of one row's dimensions as B-operand fragments: dims
// 16 kk + 8 half + (0..7)
template <int D, bool F16>
__device__ __forceinline__ void load_row_frags(const void* row, uint32_t half, bf16x8 (&f)[D / 16]) {
  const char* p = (const char*)row + half * 16;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = frag<F16>(*(const uint4*)(p + kk * 32));
}

// One LDS block stage: 32 rows x D 16-bit elements in the grouped layout.
template <int D, int I, int T>
struct BStage {
  static __device__ __forceinline__ char* ptr() {
    __shared__ __attribute__((aligned(1024))) __bf16 buf[BN * D];
    return (char*)buf;
  }
};

// Units of at most this many rows form their rows' byte offsets once per
// workgroup, into an LDS table (two maps); longer units form them per load.
constexpr int BT_ROWS = 512;
template <bool TAB>
struct RowTab {
  static __device__ __forceinline__ uint32_t* ptr() {
    __shared__ uint32_t t[TAB ? 2 * BT_ROWS : 1];
    return t;
  }
};

// One stage of a query block's row statistics: lse in slots 0..31, D in 32..63.
template <int I>
struct StatStage {
  static __device__ __forceinline__ float* ptr() {
    __shared__ __attribute__((aligned(16))) float buf[2 * BN];
    return buf;
  }
};

// Per-lane geometry of the grouped layout.
template <int D, int NW>
struct Layout {
  typedef BCfg<D, NW> C;
  // direct loads: lane i of load `ins` fills slot i of its groups
  uint32_t ld_row[C::VPW];      // row within the block
  uint32_t ld_byte[C::VPW];     // byte offset of the chunk within the row
  // row reads of chunk 2 kk + half of row l32: byte offset rd[kk % 2] + 256 (kk / 2)
  // (the swizzle only touches the low two bits of the chunk index)
  uint32_t rd[2];
  // transposing reads (lo: groups 4 jk + half, hi: + 2): byte offsets within a block
  uint32_t tr_lo, tr_hi;

  __device__ __forceinline__ void init(uint32_t lane, uint32_t wave) {
    const uint32_t half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const uint32_t ins = wave + i * NW;
      const uint32_t g = ins * C::GPI + lane / (4 * C::CPR);
      const uint32_t slot = lane % (4 * C::CPR);
      ld_row[i] = 4 * g + (slot & 3);
      ld_byte[i] = (((slot >> 2) ^ (g & 3)) << 4);
    }
    const uint32_t g = l32 >> 2, rr = l32 & 3;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      rd[kk] = 2 * (g * C::GRP + (4 * ((2 * kk + half) ^ (g & 3)) + rr) * 8);
    const uint32_t tdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const uint32_t rowq = (lane & 15) >> 2;
    const uint32_t glo = half, ghi = half + 2;
    tr_lo = 2 * (glo * C::GRP + 8 * (4 * ((tdim >> 3) ^ glo) + rowq) + (tdim & 7));
    tr_hi = 2 * (ghi * C::GRP + 8 * (4 * ((tdim >> 3) ^ ghi) + rowq) + (tdim & 7));
  }
};

// A operand from rows: 32 rows x dims 16 kk ... (lane: row l32, chunk 2 kk + half)
template <bool F16, typename Lay>
__device__ __forceinline__ bf16x8 read_rows(const char* stage, const Lay& lay, int kk) {
  return frag<F16>(*(const uint4*)(stage + lay.rd[kk & 1] + 256 * (kk >> 1)));
}

// A operand transposed: dims 32 mt + (lane % 32) x rows 16 jk + (permuted)
template <int D, bool F16, typename Lay>
__device__ __forceinline__ bf16x8 read_tr(const char* stage, const Lay& lay, int jk, int mt) {
  const char* p = stage + 2 * (4 * jk * (4 * D) + 128 * mt);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(__attribute__((address_space(3))) char*)(p + lay.tr_lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(__attribute__((address_space(3))) char*)(p + lay.tr_hi));
  // the two halves side by side: a register pairing, no arithmetic
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return frag<F16>(__builtin_bit_cast(uint4, both));
}

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

__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Store a transposed accumulator tile set: lane l32 (and l32 + 32) owns row l32,
// holding its element dim 32 mt + 8 (r / 4) + 4 half + r % 4 in acc[mt][r]; `off` is
// the row's offset under the map (kNoRow: not stored).  Each value is scaled, then
// - kAccWrite: written as fp32 to accp; kAccAdd: added to the fp32 accumulator and
//   written back; kAccFinal: added to it (if any) and written as bf16 to outp;
// - kPartWrite: written to outp as fp16 times a power of two 2^e per row, e chosen
//   so that the row's largest magnitude lies in [2^14, 2^15) (e clamped to
//   [-126, 126]), with 2^-e stored at scp[row]; kPartFinal: outp holds such a
//   part, which is added (times scp[row]) before the sum is written as bf16 to outp;
//   kPartAdd: the sum is written back as such a part, e chosen from the bound
//   2^15 scp[row] + (the row's largest new magnitude) on the sum's magnitude (the
//   row's owning lanes read the old scale before any lane writes the new one).
// scp is indexed by the row's element offset / D (the scale array has one float
// per head row of the tensor).  The rows pass through `stage` (32 rows x D / 2 fp32 =
// 64 D bytes of LDS, the wave's own) half a row at a time and go out as whole row
// segments, 16 (fp32) or 8 (16-bit) bytes per lane, so a store instruction covers
// 64 / (D / 8) rows' contiguous bytes rather than pieces of 32 rows.  Chunks are
// XOR-swizzled by row in LDS.
template <int D, bool WIDE = false>
__device__ __forceinline__ void store_rows_lds(const f32x16 (&acc)[D / 32], float scale, uint32_t lane,
                                               uint32_t mode, float* accp, __bf16* outp, uint32_t off,
                                               char* stage, float* scp = nullptr) {
  constexpr int DR = D / 2;        // fp32 dims per round
  constexpr int NCH = DR / 4;      // 16-byte chunks per staged row
  constexpr int MTR = D / 64;      // accumulator tiles per round
  constexpr int RPI = 64 / NCH;    // rows per store instruction
  const uint32_t half = lane >> 5, l32 = lane & 31;
  const bool part = mode == kPartWrite || mode == kPartFinal || mode == kPartAdd;
  // kPartWrite, kPartAdd: this row's exponent e (lanes l32 and l32 + 32 agree);
  // kPartAdd also the old part's scale, read here by the row's owners
  int32_t e_row = 0;
  float down_row = 0.f;
  if (mode == kPartWrite || mode == kPartAdd) {
    float amax = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[mt][r] * scale));
    amax = max_halves(amax);
    if (mode == kPartAdd && off != kNoRow) {
      down_row = scp[row_elems<WIDE, D>((int32_t)off) / D];
      amax += 32768.f * down_row;   // the old part's magnitudes are below 2^15 times its scale
    }
    // amax = f 2^k, f in [0.5, 1): amax 2^(15 - k) = f 2^15 lies in [2^14, 2^15)
    e_row = min(max(15 - __builtin_amdgcn_frexp_expf(amax), -126), 126);
  }
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
    for (int m = 0; m < MTR; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int mt = rd * MTR + m;
        const uint32_t ch = 8 * m + 2 * g + half;
        *(float4*)(stage + l32 * (DR * 4) + ((ch ^ (l32 & (NCH - 1))) << 4)) =
            make_float4(acc[mt][4 * g] * scale, acc[mt][4 * g + 1] * scale, acc[mt][4 * g + 2] * scale,
                        acc[mt][4 * g + 3] * scale);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the staged half rows are in LDS
    const uint32_t c = lane % NCH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const uint32_t r = i * RPI + lane / NCH;
      const uint32_t o = (uint32_t)__shfl((int)off, (int)r, 64);
      const int32_t er = __shfl(e_row, (int)r, 64);
      const float dold = __shfl(down_row, (int)r, 64);
      float4 x = *(const float4*)(stage + r * (DR * 4) + ((c ^ (r & (NCH - 1))) << 4));
      if (o != kNoRow) {
        const auto oe = row_elems<WIDE, D>((int32_t)o);
        const int d0 = DR * rd + 4 * c;
        if (part) {
          float* sp = scp + oe / D;
          if (mode == kPartWrite || mode == kPartAdd) {
            const float up = __builtin_amdgcn_ldexpf(1.f, er);
            if (mode == kPartAdd) {
              const f16x4 y = *(const f16x4*)((const _Float16*)outp + oe + d0);
              x.x = fmaf((float)y[0], dold, x.x); x.y = fmaf((float)y[1], dold, x.y);
              x.z = fmaf((float)y[2], dold, x.z); x.w = fmaf((float)y[3], dold, x.w);
            }
            f16x4 w;
            w[0] = (_Float16)(x.x * up); w[1] = (_Float16)(x.y * up);
            w[2] = (_Float16)(x.z * up); w[3] = (_Float16)(x.w * up);
            *(f16x4*)((_Float16*)outp + oe + d0) = w;
            if (rd == 0 && c == 0) *sp = __builtin_amdgcn_ldexpf(1.f, -er);
          } else {
            const float down = *sp;
            const f16x4 y = *(const f16x4*)((const _Float16*)outp + oe + d0);
            bf16x4 w;
            w[0] = (__bf16)fmaf((float)y[0], down, x.x); w[1] = (__bf16)fmaf((float)y[1], down, x.y);
            w[2] = (__bf16)fmaf((float)y[2], down, x.z); w[3] = (__bf16)fmaf((float)y[3], down, x.w);
            *(bf16x4*)(outp + oe + d0) = w;
          }
          continue;
        }
        if (mode != kAccWrite && accp) {
          const float4 y = *(const float4*)(accp + oe + d0);
          x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
        if (mode == kAccFinal) {
          bf16x4 w;
          w[0] = (__bf16)x.x; w[1] = (__bf16)x.y; w[2] = (__bf16)x.z; w[3] = (__bf16)x.w;
          *(bf16x4*)(outp + oe + d0) = w;
        } else {
          *(float4*)(accp + oe + d0) = x;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the stage is read before it is rewritten
  }
}

// ---------------------------------------------------------------- kind A: dq (and D)

template <int D, int NW, bool VF16, bool OF16, bool CUT, bool TAB, typename Args = BwdArgs, bool WIDE = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_bf16(Args a) {
  typedef BCfg<D, NW> C;
  // wide maps (row offsets in head rows) form their rows' offsets per load
  static_assert(!(WIDE && TAB), "the row tables hold 32-bit byte offsets");
  typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type boff_t;
  constexpr int BM = C::BM;
  UnitPos p;
  if (!unit_pos(a, p)) return;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t half = lane >> 5, l32 = lane & 31;
  const uint32_t L = a.L;
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, p.s);
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };
  // the row a load of row r reads: r itself, or a present row standing in for it
  auto load_row = [&](uint32_t r) -> uint32_t {
    if constexpr (CUT) return present(r) ? r : 0;
    return min(r, L - 1);
  };
  const char* qg = (const char*)a.q + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* kg = (const char*)a.k + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* vg = (const char*)a.v + 2 * a.mv.base(p.b, p.h, p.s);
  const char* og = (const char*)a.o + 2 * a.mo.base(p.b, p.h, p.s);
  const char* dg = (const char*)a.dout + 2 * a.mdo.base(p.b, p.h, p.s);

  const uint32_t q0 = p.chunk * BM + wave * 32;
  const bool active = q0 < L;
  const uint32_t qi = q0 + l32;
  const bool qok = present(qi);
  const uint32_t qr = load_row(qi);

  // query and upstream-gradient fragments; D = <dout, o> over this lane's dims,
  // unless the pass above already left D for these rows
  bf16x8 qf[D / 16], df[D / 16];
  load_row_frags<D, false>(qg + row_bytes16<WIDE, D>(a.mqk.row_off(qr)), half, qf);
  load_row_frags<D, false>(dg + row_bytes16<WIDE, D>(a.mdo.row_off(qr)), half, df);
  const size_t row_id = (size_t)p.u * L + qi;
  float dsum = 0.f;
  if (a.dsum_ready) {
    dsum = qok ? a.dsum[row_id] : 0.f;
  } else {
    const char* orow = og + row_bytes16<WIDE, D>(a.mo.row_off(qr)) + half * 16;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint4 raw = *(const uint4*)(orow + kk * 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)df[kk][e], elem<OF16>(&raw, e), dsum);
    }
    dsum = sum_halves(dsum);
  }
  // fp16 values (the global pass reads the local output): dP^T runs on fp16 MFMAs
  // with the row's dout scaled by a power of two into fp16 range (max |dout| to
  // [2^13, 2^14)), undone on the fp32 product, so V needs no conversion per block
  typedef _Float16 f16x8l __attribute__((ext_vector_type(8)));
  f16x8l dh[VF16 ? D / 16 : 1];
  float dp_scale = 1.f;
  if constexpr (VF16) {
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf((float)df[kk][e]));
    mx = max_halves(mx);
    int ex = 0;
    if (mx > 0.f) (void)frexpf(mx, &ex);   // mx = f 2^ex, f in [0.5, 1)
    const float up = ldexpf(1.f, 14 - ex);
    dp_scale = ldexpf(1.f, ex - 14);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) dh[kk][e] = (_Float16)((float)df[kk][e] * up);
  }
  const float lse = qok ? a.lse[row_id] : 0.f;
  if (!a.dsum_ready && qok && half == 0) a.dsum[row_id] = dsum;

  Layout<D, NW> lay;
  lay.init(lane, wave);
  const uint32_t nkb = (L + BN - 1) / BN;
  uint32_t* tab = RowTab<TAB>::ptr();   // K rows, then V rows (byte offsets)
  if constexpr (TAB) {
    for (uint32_t r = tid; r < nkb * BN; r += 64 * NW) {
      const uint32_t rr = load_row(r);
      tab[r] = bytes16(a.mqk.row_off(rr));
      tab[BT_ROWS + r] = bytes16(a.mv.row_off(rr));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the table is written
    __builtin_amdgcn_s_barrier();
  }
  auto issue = [&](uint32_t kb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    char* ks = BStage<D, ST, 0>::ptr();
    char* vs = BStage<D, ST, 1>::ptr();
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const uint32_t ins = wave + i * NW;
      boff_t ko, vo;
      if constexpr (TAB) {
        ko = tab[kb * BN + lay.ld_row[i]];
        vo = tab[BT_ROWS + kb * BN + lay.ld_row[i]];
      } else {
        const uint32_t r = load_row(kb * BN + lay.ld_row[i]);
        ko = row_bytes16<WIDE, D>(a.mqk.row_off(r));
        vo = row_bytes16<WIDE, D>(a.mv.row_off(r));
      }
      __builtin_amdgcn_global_load_lds((const void*)(kg + ko + lay.ld_byte[i]),
                                       (lds_void_t*)(ks + ins * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vg + vo + lay.ld_byte[i]),
                                       (lds_void_t*)(vs + ins * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
  const float c = a.c;

  // three stages: block kb sits in stage kb % 3 and is requested two steps ahead.
  // ALL: block kb + 2 exists (known at compile time, so the main loop's steps
  // have no conditional loads and the compiler's waits before the LDS reads stay
  // per stage instead of draining every load)
  auto step = [&](uint32_t kb, auto st_tag, auto all_tag) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool ALL = decltype(all_tag)::value;
    const bool has2 = ALL || kb + 2 < nkb;
    if (has2) issue(kb + 2, std::integral_constant<int, (ST + 2) % 3>{});
    if (active) {
      const char* ks = BStage<D, ST, 0>::ptr();
      const char* vs = BStage<D, ST, 1>::ptr();
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sc = mfma(read_rows<false>(ks, lay, kk), qf[kk], sc);
        if constexpr (VF16)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8l, *(const uint4*)(vs + lay.rd[kk & 1] + 256 * (kk >> 1))), dh[kk], dp, 0, 0, 0);
        else
          dp = mfma(read_rows<false>(vs, lay, kk), df[kk], dp);
      }
      // present keys of the block: bit j for key kb * 32 + j, then this half's bits
      uint32_t km = 0xffffffffu;
      if constexpr (CUT) {
        km = (uint32_t)__ballot(present(kb * BN + l32));
      } else if ((kb + 1) * BN > L) {
        km = (1u << (L - kb * BN)) - 1u;   // fewer than 32 keys left
      }
      bf16x8 db[2];
      if (km == 0xffffffffu) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          db[r / 8][r % 8] = (__bf16)(__builtin_amdgcn_exp2f(fmaf(sc[r], c, -lse)) * fmaf(dp[r], dp_scale, -dsum));
      } else {
        km >>= 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pij = __builtin_amdgcn_ubfe(km, 8 * (r / 4) + (r % 4), 1) ? __builtin_amdgcn_exp2f(fmaf(sc[r], c, -lse)) : 0.f;
          db[r / 8][r % 8] = (__bf16)(pij * fmaf(dp[r], dp_scale, -dsum));
        }
      }
#pragma unroll
      for (int jk = 0; jk < 2; ++jk)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) acc[mt] = mfma(read_tr<D, false>(ks, lay, jk, mt), db[jk], acc[mt]);
    }
    // this wave's loads of block kb + 1 have landed (those of kb + 2 may be in
    // flight); the barrier publishes them and retires stage ST's readers
    if (ALL) wait_vmcnt<2 * C::VPW>();
    else if (has2) wait_vmcnt<2 * C::VPW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };

  issue(0, std::integral_constant<int, 0>{});
  if (nkb > 1) issue(1, std::integral_constant<int, 1>{});
  // the prologue's row loads and block 0 have landed
  if (nkb > 1) wait_vmcnt<2 * C::VPW>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  uint32_t kb = 0;
  for (; kb + 5 <= nkb; kb += 3) {
    step(kb, std::integral_constant<int, 0>{}, std::true_type{});
    step(kb + 1, std::integral_constant<int, 1>{}, std::true_type{});
    step(kb + 2, std::integral_constant<int, 2>{}, std::true_type{});
  }
  for (; kb + 3 <= nkb; kb += 3) {
    step(kb, std::integral_constant<int, 0>{}, std::false_type{});
    step(kb + 1, std::integral_constant<int, 1>{}, std::false_type{});
    step(kb + 2, std::integral_constant<int, 2>{}, std::false_type{});
  }
  if (kb < nkb) step(kb, std::integral_constant<int, 0>{}, std::false_type{});
  if (kb + 1 < nkb) step(kb + 1, std::integral_constant<int, 1>{}, std::false_type{});

  // (every wave is past the last step's barrier: the stages are free, and wave w
  // stages its stores in one of them)
  if (active) {
    char* st = wave == 0 ? BStage<D, 0, 0>::ptr()
             : wave == 1 ? BStage<D, 1, 0>::ptr()
             : wave == 2 ? BStage<D, 2, 0>::ptr() : BStage<D, 0, 1>::ptr();
    const int64_t base = a.mdq.base(p.b, p.h, p.s);
    store_rows_lds<D, WIDE>(acc, a.scale, lane, a.final_pass, a.dq_acc ? a.dq_acc + base : nullptr,
                            a.final_pass != kAccWrite && a.final_pass != kAccAdd ? (__bf16*)a.dq + base : nullptr,
                            qok ? (uint32_t)a.mdq.row_off(qi) : kNoRow, st, a.dq_sc ? a.dq_sc + base / D : nullptr);
  }
}

// ---------------------------------------------------------------- kind B: dk, dv

template <int D, int NW, bool VF16, bool CUT, bool TAB, typename Args = BwdArgs, bool WIDE = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_bf16(Args a) {
  typedef BCfg<D, NW> C;
  static_assert(!(WIDE && TAB), "the row tables hold 32-bit byte offsets");
  typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type boff_t;
  constexpr int BM = C::BM;
  UnitPos p;
  if (!unit_pos(a, p)) return;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t half = lane >> 5, l32 = lane & 31;
  const uint32_t L = a.L;
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, p.s);
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };
  auto load_row = [&](uint32_t r) -> uint32_t {
    if constexpr (CUT) return present(r) ? r : 0;
    return min(r, L - 1);
  };
  const char* qg = (const char*)a.q + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* kg = (const char*)a.k + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* vg = (const char*)a.v + 2 * a.mv.base(p.b, p.h, p.s);
  const char* dg = (const char*)a.dout + 2 * a.mdo.base(p.b, p.h, p.s);

  const uint32_t k0 = p.chunk * BM + wave * 32;
  const bool active = k0 < L;
  const uint32_t kj = k0 + l32;
  const bool kok = present(kj);
  const uint32_t kr = load_row(kj);
  bf16x8 kf[D / 16];
  load_row_frags<D, false>(kg + row_bytes16<WIDE, D>(a.mqk.row_off(kr)), half, kf);
  // the workgroup's own V rows, bf16, in LDS: chunk c of row r at slot c ^ (r % CPR)
  // (read as the B operand of dP, one 16-byte chunk per lane, conflict-free);
  // holding them in registers instead would not leave room for both accumulators
  __shared__ __attribute__((aligned(1024))) __bf16 vown[BM * D];
  {
    constexpr int PER = BM * C::CPR / (64 * NW);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t ch = tid + 64 * NW * i;
      const uint32_t r = ch / C::CPR, cc = ch % C::CPR;
      const uint32_t vr = load_row(p.chunk * BM + r);
      const uint4 raw = *(const uint4*)(vg + row_bytes16<WIDE, D>(a.mv.row_off(vr)) + 16 * cc);
      *(bf16x8*)((char*)vown + r * D * 2 + ((cc ^ (r & (C::CPR - 1))) << 4)) = frag<VF16>(raw);
    }
  }
  const char* vrow_lds = (const char*)vown + (wave * 32 + l32) * D * 2;
  const uint32_t vxor = l32 & (C::CPR - 1);

  Layout<D, NW> lay;
  lay.init(lane, wave);
  const size_t unit_rows = (size_t)p.u * L;
  const uint32_t nqb = (L + BN - 1) / BN;
  uint32_t* tab = RowTab<TAB>::ptr();   // Q rows, then dout rows (byte offsets)
  if constexpr (TAB) {
    for (uint32_t r = tid; r < nqb * BN; r += 64 * NW) {
      const uint32_t rr = load_row(r);
      tab[r] = bytes16(a.mqk.row_off(rr));
      tab[BT_ROWS + r] = bytes16(a.mdo.row_off(rr));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the table is written
    __builtin_amdgcn_s_barrier();
  }
  auto issue = [&](uint32_t qb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    char* qs = BStage<D, ST, 2>::ptr();
    char* ds = BStage<D, ST, 3>::ptr();
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const uint32_t ins = wave + i * NW;
      boff_t qo, dof;
      if constexpr (TAB) {
        qo = tab[qb * BN + lay.ld_row[i]];
        dof = tab[BT_ROWS + qb * BN + lay.ld_row[i]];
      } else {
        const uint32_t r = load_row(qb * BN + lay.ld_row[i]);
        qo = row_bytes16<WIDE, D>(a.mqk.row_off(r));
        dof = row_bytes16<WIDE, D>(a.mdo.row_off(r));
      }
      __builtin_amdgcn_global_load_lds((const void*)(qg + qo + lay.ld_byte[i]),
                                       (lds_void_t*)(qs + ins * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dg + dof + lay.ld_byte[i]),
                                       (lds_void_t*)(ds + ins * 1024), 16, 0, 0);
    }
    // the block's row statistics by one more direct load (lane i < 32: lse of row
    // i, lane 32 + i: its D); every wave issues it, so the load counts and waits
    // are the same in all waves (the duplicate writes carry the same values).
    // Rows past the end or absent read a present row; the query mask drops them.
    {
      const uint32_t rr = load_row(qb * BN + l32);
      const float* src = (half ? (const float*)a.dsum : a.lse) + unit_rows + rr;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)StatStage<ST>::ptr(), 4, 0, 0);
    }
  };

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dka[mt][r] = 0.f; dva[mt][r] = 0.f; }
  const float c = a.c;

  // two stages: the next block is requested before the current one is used.
  // ALL: the next block exists (known at compile time: no conditional loads in the
  // main loop, so the compiler's waits before the LDS reads stay per stage)
  auto step = [&](uint32_t qb, auto st_tag, auto all_tag) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool ALL = decltype(all_tag)::value;
    if (ALL || qb + 1 < nqb) issue(qb + 1, std::integral_constant<int, ST ^ 1>{});
    if (active) {
      const char* qs = BStage<D, ST, 2>::ptr();
      const char* ds = BStage<D, ST, 3>::ptr();
      const float* stat = StatStage<ST>::ptr();
      // present queries of the block: bit j for query qb * 32 + j, then this half's
      uint32_t qm = 0xffffffffu;
      if constexpr (CUT) {
        qm = (uint32_t)__ballot(present(qb * BN + l32));
      } else if ((qb + 1) * BN > L) {
        qm = (1u << (L - qb * BN)) - 1u;   // fewer than 32 queries left
      }
      const bool all_q = qm == 0xffffffffu;
      qm >>= 4 * half;
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sc = mfma(read_rows<false>(qs, lay, kk), kf[kk], sc);
        dp = mfma(read_rows<false>(ds, lay, kk),
                  *(const bf16x8*)(vrow_lds + (((uint32_t)(2 * kk) + half) ^ vxor) * 16), dp);
      }
      bf16x8 pb[2], sb[2];
      if (!all_q) {
        // queries past the end or absent: their scores become -inf (weight 0)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!__builtin_amdgcn_ubfe(qm, 8 * (r / 4) + (r % 4), 1)) sc[r] = -INFINITY;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // queries 8 g + 4 half + (0..3) of the block
        const float4 ls = *(const float4*)&stat[8 * g + 4 * half];
        const float4 dd = *(const float4*)&stat[BN + 8 * g + 4 * half];
        const float lv[4] = {ls.x, ls.y, ls.z, ls.w};
        const float dv4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pij = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -lv[e]));
          pb[r / 8][r % 8] = (__bf16)pij;
          sb[r / 8][r % 8] = (__bf16)(pij * (dp[r] - dv4[e]));
        }
      }
#pragma unroll
      for (int jk = 0; jk < 2; ++jk)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          dva[mt] = mfma(read_tr<D, false>(ds, lay, jk, mt), pb[jk], dva[mt]);
          dka[mt] = mfma(read_tr<D, false>(qs, lay, jk, mt), sb[jk], dka[mt]);
        }
    }
    // the next block has landed; the barrier publishes it and retires stage ST
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };

  issue(0, std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0);   // block 0 and the own V rows (LDS stores) are in place
  __builtin_amdgcn_s_barrier();
  uint32_t qb = 0;
  for (; qb + 3 <= nqb; qb += 2) {
    step(qb, std::integral_constant<int, 0>{}, std::true_type{});
    step(qb + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  if (qb < nqb) step(qb, std::integral_constant<int, 0>{}, std::false_type{});
  if (qb + 1 < nqb) step(qb + 1, std::integral_constant<int, 1>{}, std::false_type{});

  // D of the pass below for this wave's value rows, <dv_j, v_j>, with dv_j rounded
  // to bf16 as it is stored (the pass below forms its products from those values)
  // and v_j the own row in LDS, as rounded for the products; read from LDS before
  // the stores below reuse those rows
  if (a.dsum_next && active) {
    float dn = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // dims 32 mt + 8 g + 4 half + (0..3): chunk 4 mt + g, elements 4 half + (0..3)
        const uint2 raw = *(const uint2*)(vrow_lds + (((uint32_t)(4 * mt + g) ^ vxor) << 4) + 8 * half);
        const bf16x4 vv = __builtin_bit_cast(bf16x4, raw);
#pragma unroll
        for (int e = 0; e < 4; ++e) dn = fmaf((float)(__bf16)dva[mt][4 * g + e], (float)vv[e], dn);
      }
    dn = sum_halves(dn);
    const uint32_t bh = p.b * a.heads + p.h;
    if (kok && half == 0) a.dsum_next[((size_t)kj * a.BH + bh) * a.U + p.s] = dn;
  }
  // (every wave is past the last step's barrier: wave w stages its stores in its
  // own 32 rows of the V block)
  if (active) {
    char* st = (char*)vown + wave * 32 * D * 2;
    const int64_t kbase = a.mdk.base(p.b, p.h, p.s), vbase = a.mdv.base(p.b, p.h, p.s);
    store_rows_lds<D, WIDE>(dka, a.scale, lane, a.final_pass, a.dk_acc ? a.dk_acc + kbase : nullptr,
                            a.final_pass != kAccWrite && a.final_pass != kAccAdd ? (__bf16*)a.dk + kbase : nullptr,
                      kok ? (uint32_t)a.mdk.row_off(kj) : kNoRow, st, a.dk_sc ? a.dk_sc + kbase / D : nullptr);
    store_rows_lds<D, WIDE>(dva, 1.f, lane, kAccFinal, nullptr, (__bf16*)a.dv + vbase,
                      kok ? (uint32_t)a.mdv.row_off(kj) : kNoRow, st);
  }
}

// ---------------------------------------------------------------- units of at most 64 rows

// A whole unit of at most 64 rows in one two-wave workgroup: S and dP are formed
// once and feed all three gradients (five products instead of the seven of kinds A
// and B, and every row read once).  The unit's Q, dout and K rows sit in LDS
// (grouped layout, two blocks each); wave w owns keys 32 w .. 32 w + 31 as in
// kind B, with its V rows in registers (S = Q K^T, dP = dout V^T; dv^T += dout^T P,
// dk^T += Q^T dS), and keeps its dS in registers.  Once every wave is done with
// the dout blocks, the dS rows (queries) go to their place, and wave w forms dq^T
// of query block w as K^T dS^T (A = K^T by the transposing read, B = dS^T rows in
// the key order of that read).  D = <dout, o> of the unit's rows is formed in the
// prologue.  LDS: 48 KB at head dim 128, so three workgroups share a CU.
constexpr int SMALL_ROWS = 64;

template <int D, bool VF16, bool OF16, typename Args>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_small_bf16(Args a) {
  constexpr int NW = 2;
  typedef BCfg<D, NW> C;
  // dS row pitch (16-bit elements): 64 keys, padded where the dout block has room
  constexpr int PITCH = BN * D >= BN * (2 * BN + 8) ? 2 * BN + 8 : 2 * BN;
  static_assert(BN * PITCH <= BN * D, "a block of dS rows fits a dout block");
  UnitPos p;
  if (!unit_pos(a, p)) return;   // one workgroup per unit (nchunks = 1)
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t half = lane >> 5, l32 = lane & 31;
  const uint32_t L = a.L;   // 1 .. 64
  auto load_row = [&](uint32_t r) -> uint32_t { return min(r, L - 1); };
  const char* qg = (const char*)a.q + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* kg = (const char*)a.k + 2 * a.mqk.base(p.b, p.h, p.s);
  const char* vg = (const char*)a.v + 2 * a.mv.base(p.b, p.h, p.s);
  const char* og = (const char*)a.o + 2 * a.mo.base(p.b, p.h, p.s);
  const char* dg = (const char*)a.dout + 2 * a.mdo.base(p.b, p.h, p.s);
  const uint32_t nb = (L + BN - 1) / BN;   // 1 or 2 blocks

  Layout<D, NW> lay;
  lay.init(lane, wave);
  // every row of the unit: Q, dout and K blocks by direct loads (rows past the
  // end read the last row; their scores are masked and their dS is zero)
  auto issue = [&](uint32_t b, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const uint32_t ins = wave + i * NW;
      const uint32_t r = load_row(b * BN + lay.ld_row[i]);
      const uint32_t qo = bytes16(a.mqk.row_off(r)) + lay.ld_byte[i];
      __builtin_amdgcn_global_load_lds((const void*)(qg + qo), (lds_void_t*)(BStage<D, ST, 2>::ptr() + ins * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(kg + qo), (lds_void_t*)(BStage<D, ST, 4>::ptr() + ins * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dg + bytes16(a.mdo.row_off(r)) + lay.ld_byte[i]),
                                       (lds_void_t*)(BStage<D, ST, 3>::ptr() + ins * 1024), 16, 0, 0);
    }
  };
  issue(0, std::integral_constant<int, 0>{});
  if (nb > 1) issue(1, std::integral_constant<int, 1>{});

  const uint32_t rj = wave * 32 + l32;   // this lane's key (dk, dv) and query (dq)
  const bool rok = rj < L;
  const uint32_t rr = load_row(rj);
  // the own V rows (B operands of dP), bf16
  bf16x8 vf[D / 16];
  load_row_frags<D, VF16>(vg + bytes16(a.mv.row_off(rr)), half, vf);
  // row statistics of the unit: lse and D = <dout, o> (wave w: rows 32 w + l32)
  __shared__ __attribute__((aligned(16))) float stat_l[SMALL_ROWS];
  __shared__ __attribute__((aligned(16))) float stat_d[SMALL_ROWS];
  {
    const char* drow = dg + bytes16(a.mdo.row_off(rr)) + half * 16;
    const char* orow = og + bytes16(a.mo.row_off(rr)) + half * 16;
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint4 dr = *(const uint4*)(drow + kk * 32);
      const uint4 orw = *(const uint4*)(orow + kk * 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf(elem<false>(&dr, e), elem<OF16>(&orw, e), dsum);
    }
    dsum = sum_halves(dsum);
    if (half == 0) stat_d[rj] = rok ? dsum : 0.f;
    else stat_l[rj] = rok ? a.lse[(size_t)p.u * L + rj] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0);   // every direct load and LDS store is in place
  __builtin_amdgcn_s_barrier();

  const bool active = wave * 32 < L;
  const char* kown = wave == 0 ? BStage<D, 0, 4>::ptr() : BStage<D, 1, 4>::ptr();
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dka[mt][r] = 0.f; dva[mt][r] = 0.f; }
  bf16x8 sbk[2][2];   // dS of each query block (S layout: this lane's key)
  const float c = a.c;
  auto step = [&](uint32_t qb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const char* qs = BStage<D, ST, 2>::ptr();
    const char* ds = BStage<D, ST, 3>::ptr();
    f32x16 sc, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      sc = mfma(read_rows<false>(qs, lay, kk), read_rows<false>(kown, lay, kk), sc);
      dp = mfma(read_rows<false>(ds, lay, kk), vf[kk], dp);
    }
    // queries past the end: weight 0
    uint32_t qm = 0xffffffffu;
    if ((qb + 1) * BN > L) qm = (1u << (L - qb * BN)) - 1u;
    qm >>= 4 * half;
    bf16x8 pb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // queries 8 g + 4 half + (0..3) of the block
      const float4 ls = *(const float4*)&stat_l[qb * BN + 8 * g + 4 * half];
      const float4 dd = *(const float4*)&stat_d[qb * BN + 8 * g + 4 * half];
      const float lv[4] = {ls.x, ls.y, ls.z, ls.w};
      const float dv4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const bool qin = __builtin_amdgcn_ubfe(qm, 8 * g + e, 1);
        const float pij = qin ? __builtin_amdgcn_exp2f(fmaf(sc[r], c, -lv[e])) : 0.f;
        pb[r / 8][r % 8] = (__bf16)pij;
        sbk[ST][r / 8][r % 8] = (__bf16)(pij * (dp[r] - dv4[e]));
      }
    }
#pragma unroll
    for (int jk = 0; jk < 2; ++jk)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        dva[mt] = mfma(read_tr<D, false>(ds, lay, jk, mt), pb[jk], dva[mt]);
        dka[mt] = mfma(read_tr<D, false>(qs, lay, jk, mt), sbk[ST][jk], dka[mt]);
      }
  };
  if (active) {
    step(0, std::integral_constant<int, 0>{});
    if (nb > 1) step(1, std::integral_constant<int, 1>{});
  }
  // every wave is done with the Q and dout blocks: the dout blocks take the dS rows
  // of their query block ([query][key], PITCH apart; keys past the end take no
  // part), and each wave stages its stores through its own Q block
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  __bf16* ds0 = (__bf16*)BStage<D, 0, 3>::ptr();
  __bf16* ds1 = (__bf16*)BStage<D, 1, 3>::ptr();
  char* own_stage = wave == 0 ? BStage<D, 0, 2>::ptr() : BStage<D, 1, 2>::ptr();
  if (active) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t q = 8 * (r / 4) + 4 * half + (r % 4);
      ds0[q * PITCH + rj] = rok ? sbk[0][r / 8][r % 8] : (__bf16)0.f;
      if (nb > 1) ds1[q * PITCH + rj] = rok ? sbk[1][r / 8][r % 8] : (__bf16)0.f;
    }
    const int64_t kb0 = a.mdk.base(p.b, p.h, p.s), vb0 = a.mdv.base(p.b, p.h, p.s);
    store_rows_lds<D>(dka, a.scale, lane, a.final_pass, a.dk_acc ? a.dk_acc + kb0 : nullptr,
                      a.final_pass != kAccWrite && a.final_pass != kAccAdd ? (__bf16*)a.dk + kb0 : nullptr,
                      rok ? (uint32_t)a.mdk.row_off(rj) : kNoRow, own_stage,
                      a.dk_sc ? a.dk_sc + kb0 / D : nullptr);
    store_rows_lds<D>(dva, 1.f, lane, kAccFinal, nullptr, (__bf16*)a.dv + vb0,
                      rok ? (uint32_t)a.mdv.row_off(rj) : kNoRow, own_stage);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's dS rows are written
  __builtin_amdgcn_s_barrier();
  if (!active) return;

  // dq^T of query block `wave` over the unit's keys: B = dS^T (this lane's query
  // row, keys 16 jk + 4 half + (0..3) and 16 jk + 8 + 4 half + (0..3) of each key
  // block: the row order of the transposing read of K)
  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
  const __bf16* qrow = (wave == 0 ? ds0 : ds1) + l32 * PITCH + 4 * half;
  auto dq_block = [&](uint32_t kb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    const char* ks = BStage<D, ST, 4>::ptr();
#pragma unroll
    for (int jk = 0; jk < 2; ++jk) {
      const uint2 lo = *(const uint2*)(qrow + kb * BN + 16 * jk);
      const uint2 hi = *(const uint2*)(qrow + kb * BN + 16 * jk + 8);
      const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) acc[mt] = mfma(read_tr<D, false>(ks, lay, jk, mt), b, acc[mt]);
    }
  };
  dq_block(0, std::integral_constant<int, 0>{});
  if (nb > 1) dq_block(1, std::integral_constant<int, 1>{});
  const int64_t qb0 = a.mdq.base(p.b, p.h, p.s);
  store_rows_lds<D>(acc, a.scale, lane, a.final_pass, a.dq_acc ? a.dq_acc + qb0 : nullptr,
                    a.final_pass != kAccWrite && a.final_pass != kAccAdd ? (__bf16*)a.dq + qb0 : nullptr,
                    rok ? (uint32_t)a.mdq.row_off(rj) : kNoRow, own_stage, a.dq_sc ? a.dq_sc + qb0 / D : nullptr);
}

template <int D, int NW, bool VF16, bool OF16, typename Args>
hipError_t launch(const Args& a, bool kind_b, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)((a.units + 7) / 8) * 8 * a.nchunks;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 grid((uint32_t)blocks), block(64 * NW);
  if constexpr (std::is_same<Args, BwdArgs>::value) {
    if (a.row_unit > 1) {
      // wide maps: no row tables; the host marks every wide call as cut (on a whole
      // tiling every row is present)
      if (!a.cut.on) return hipErrorInvalidValue;
      if (kind_b) hipLaunchKernelGGL((bwd_dkv_bf16<D, NW, VF16, true, false, BwdArgs, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((bwd_dq_bf16<D, NW, VF16, OF16, true, false, BwdArgs, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
    // cut tilings: presence is tested per block (one ballot), with or without the tables
    if (a.cut.on) {
      const bool tab = a.L <= BT_ROWS;
      if (kind_b) {
        if (tab) hipLaunchKernelGGL((bwd_dkv_bf16<D, NW, VF16, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((bwd_dkv_bf16<D, NW, VF16, true, false>), grid, block, 0, stream, a);
      } else {
        if (tab) hipLaunchKernelGGL((bwd_dq_bf16<D, NW, VF16, OF16, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((bwd_dq_bf16<D, NW, VF16, OF16, true, false>), grid, block, 0, stream, a);
      }
      return hipGetLastError();
    }
  } else if (a.cut.on || a.row_unit > 1) {
    return hipErrorInvalidValue;
  }
  if (kind_b) {
    if (a.L <= BT_ROWS)
      hipLaunchKernelGGL((bwd_dkv_bf16<D, NW, VF16, false, true, Args>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dkv_bf16<D, NW, VF16, false, false, Args>), grid, block, 0, stream, a);
  } else {
    if (a.L <= BT_ROWS)
      hipLaunchKernelGGL((bwd_dq_bf16<D, NW, VF16, OF16, false, true, Args>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_bf16<D, NW, VF16, OF16, false, false, Args>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

// Waves per workgroup: 2 for units of at most 64 rows (half of a 4-wave
// workgroup would idle on them), else 4.
template <bool VF16, bool OF16, typename Args>
hipError_t launch_nw(Args a, int head_dim, bool kind_b, hipStream_t stream) {
  const int nw = a.L <= 64 ? 2 : 4;
  a.nchunks = (a.L + 32 * nw - 1) / (32 * nw);
  if (head_dim == 128)
    return nw == 2 ? launch<128, 2, VF16, OF16>(a, kind_b, stream) : launch<128, 4, VF16, OF16>(a, kind_b, stream);
  if (head_dim == 64)
    return nw == 2 ? launch<64, 2, VF16, OF16>(a, kind_b, stream) : launch<64, 4, VF16, OF16>(a, kind_b, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_bf16(BwdArgs a, int head_dim, BwdTypes t, bool kind_b, hipStream_t stream) {
  if (t.v_f16 && !t.o_f16) return launch_nw<true, false>(a, head_dim, kind_b, stream);
  if (!t.v_f16 && t.o_f16) return launch_nw<false, true>(a, head_dim, kind_b, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16_k(BwdArgsK a, int head_dim, bool kind_b, hipStream_t stream) {
  return launch_nw<true, true>(a, head_dim, kind_b, stream);
}

namespace {
template <bool VF16, bool OF16, typename Args>
hipError_t launch_small(Args a, int head_dim, hipStream_t stream) {
  if (a.L > SMALL_ROWS || a.cut.on) return hipErrorInvalidValue;
  if (a.row_unit > 1) return hipErrorInvalidValue;   // narrow maps only
  a.nchunks = 1;
  const uint64_t blocks = (uint64_t)((a.units + 7) / 8) * 8;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (head_dim == 128)
    hipLaunchKernelGGL((bwd_small_bf16<128, VF16, OF16, Args>), dim3((uint32_t)blocks), dim3(128), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((bwd_small_bf16<64, VF16, OF16, Args>), dim3((uint32_t)blocks), dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
}  // namespace

bool bwd_bf16_fused(uint32_t L, bool cut) { return L <= SMALL_ROWS && !cut; }

hipError_t launch_bwd_bf16_small(BwdArgs a, int head_dim, BwdTypes t, hipStream_t stream) {
  if (t.v_f16 && !t.o_f16) return launch_small<true, false>(a, head_dim, stream);
  if (!t.v_f16 && t.o_f16) return launch_small<false, true>(a, head_dim, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16_small_k(BwdArgsK a, int head_dim, hipStream_t stream) {
  return launch_small<true, true>(a, head_dim, stream);
}

}  // namespace squad
