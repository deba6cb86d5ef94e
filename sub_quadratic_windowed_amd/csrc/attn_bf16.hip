// attn_bf16.hip - the 16-bit attention engine behind both SQuad passes (gfx950 MFMA).
//
// One workgroup runs one query chunk (32 rows per wave) of one unit (a window in
// the local pass, an offset group in the global pass) against all of the unit's
// keys, streamed through LDS in blocks of 32 keys with an online softmax.  The
// standard softmax of both passes (technical summary, "1. SQuad-Attention
// Operator") is computed exactly: row max, exp2 of the shifted logits, row sum and
// a final division, in fp32.
//
// Products run on 32x32x16 MFMAs with fp32 accumulation:
//   S^T = K * Q^T   (A = 32 keys x 16 dims read from LDS, B = Q^T held in registers)
//   O^T = V^T * P^T (A = V^T read from LDS with ds_read_b64_tr_b16, B = P^T in registers)
// Computing the transposes puts one query per lane (lane % 32), so the softmax row
// statistics are per-lane scalars; the two 32-lane halves of a wave meet once per
// block.  The C/D layout of the 32x32 MFMA gives lane l, register r the element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32); P^T leaves the S^T registers in the
// k-slot order the second MFMA consumes when V^T is read with the matching key
// permutation, so P never moves between lanes.
//
// Data movement (measured on gfx950: 64 four-byte LDS banks, 256 B per clock):
//   * K rows go global -> LDS directly as well, 16-byte chunk c of row r at slot
//     c ^ (r % CPR) of the row (an XOR swizzle, CPR = chunks per row), and the A
//     operand is read as two ds_read_b64 per lane (two-way bank conflicts: the 32
//     rows a read touches share 16 slot columns).  Three K stages, two blocks ahead,
//     with no staging registers.
//   * V rows go global -> LDS directly (global_load_lds, 16 B per lane).  Each
//     group of four rows is stored chunk-interleaved: 16-byte chunk c of row r sits
//     at slot 4*c + r%4 of its group, so the four rows a transposing read touches
//     cover 16 consecutive slots (all 64 banks) and one direct load fills whole
//     groups with no idle lanes.  Three V stages, so each block's values are
//     requested two blocks ahead.
//   * Q rows are loaded straight into the B-operand registers once.
//   * The output is staged through LDS and stored as whole 16-byte chunks per row.
// Rows past the end of a unit read the unit's last row (their logits are masked to
// -inf, so they carry zero weight) and are never stored.
//
// Address work: for units of at most TABLE_ROWS rows every row's byte offset is
// formed once per workgroup into an LDS table (padded to whole blocks with the last
// row), so locating a block's rows is one LDS read and one add per load; the direct
// loads take a uniform base plus a 32-bit byte offset, and the K reads a per-lane
// offset with the stage's LDS address as the instruction's immediate.  The
// two 32-lane halves of a wave combine their row statistics with one lane-half swap
// (v_permlane32_swap) rather than an LDS round trip.
//
// The softmax keeps a reference maximum that is raised only when a block's maximum
// exceeds it by more than 2^8 in the exp2 domain; until then the weights are
// exp2(logit - reference) <= 256, well inside fp16/bf16 range, and the accumulator
// needs no rescaling.  The row sum adds the weights as rounded for the products
// (two per v_dot2 instruction), so the normalised weights of a row sum to one
// exactly as applied; it divides the accumulator out at the end.
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
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BN = 32;              // keys per block
constexpr float RESCALE_TAU = 8.f;  // log2 headroom before the reference max is raised
constexpr int TABLE_ROWS = 512;     // units of at most this many rows keep their row offsets in LDS

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

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most 2 * n direct loads (this wave's K and V loads of the newest
// block) are outstanding; n is wave-uniform and at most 4.
__device__ __forceinline__ void wait_newest(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<2>(); break;
    case 2: wait_vmcnt<4>(); break;
    case 3: wait_vmcnt<6>(); break;
    default: wait_vmcnt<8>(); break;
  }
}

// the value of lane l ^ 32, combined with this lane's: one swap of the two 32-lane halves
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int shfl(int x, int src) { return __shfl(x, src, 64); }

// sum of 16 rounded weights (two 8-element vectors) added to acc, two per
// instruction, each accumulating straight into the running sum
__device__ __forceinline__ float row_sum(const bf16x8 (&pb)[2], float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const b2 x = {pb[h][2 * e], pb[h][2 * e + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
    }
  return acc;
}
__device__ __forceinline__ float row_sum(const f16x8 (&pb)[2], float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const h2 x = {pb[h][2 * e], pb[h][2 * e + 1]};
      acc = __builtin_amdgcn_fdot2(x, one, acc, false);
    }
  return acc;
}

template <int D, int NW>
struct Cfg {
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int VGRP = 4 * D;                  // elements of one 4-row V group
  static constexpr int VINS = BN * CPR / 64;          // direct loads per K (or V) block
  static constexpr int VPW = (VINS + NW - 1) / NW;    // ... at most per wave
  static constexpr int GPI = 64 / (4 * CPR);          // 4-row groups per direct load
  static constexpr int KRPI = 64 / CPR;               // K rows per direct load
  static_assert((BN * D * 2) % 1024 == 0, "stages must be whole 1 KB direct-load blocks");
  static_assert(VINS * 64 == BN * CPR, "K/V staging split");
};

// One LDS stage of K (or V): 32 rows x D 16-bit elements.  Each stage is its own
// __shared__ object so the compiler can tell the stage being read from the stages
// whose direct loads are still in flight (no blanket vmcnt(0) before every read).
template <int D, int I>
struct Stage {
  static __device__ __forceinline__ __bf16* k() {
    __shared__ __attribute__((aligned(1024))) __bf16 buf[BN * D];
    return buf;
  }
  static __device__ __forceinline__ __bf16* v() {
    __shared__ __attribute__((aligned(1024))) __bf16 buf[BN * D];
    return buf;
  }
};

// The 16 score-register bits of lane half h for one 32-row block whose presence
// word has bit j set when row j is present: register r holds row 8*(r/4) + 4*h + r%4
// (the MFMA output layout), i.e. the nibbles at 4*h, 8 + 4*h, 16 + 4*h, 24 + 4*h.
__device__ __forceinline__ uint32_t half_bits(uint32_t rows, uint32_t h) {
  uint32_t x = (rows >> (4 * h)) & 0x0f0f0f0fu;
  x = (x | (x >> 4)) & 0x00ff00ffu;
  x = (x | (x >> 8)) & 0x0000ffffu;
  return x;
}

// CUT: the grid is not a whole number of tiles; absent rows (the far edges' cut
// tiles) are neither keys nor stored queries.  With the row tables (TAB) their
// presence bits are formed once per workgroup into LDS; without them, for each key
// block one step ahead, with one ballot.
template <int D, int NW, typename VT, typename OT, bool TAB, bool CUT = false, typename Args = AttnArgs,
          bool WIDE = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void attn16_kernel(Args a) {
  typedef Cfg<D, NW> C;
  // wide maps (row offsets in head rows) form their rows' offsets per load
  static_assert(!(WIDE && TAB), "the row tables hold 32-bit byte offsets");
  typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type boff_t;
  typedef typename Vec<VT>::x8 vx8;
  typedef typename Vec<VT>::x4 vx4;
  typedef typename Vec<OT>::x4 ox4;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const uint32_t q0 = chunk * C::BM + wave * 32;   // first query row of this wave
  const bool active = q0 < L;
  UnitDigits ud;
  if constexpr (CUT) ud = cut_unit_digits(a, s);
  // row r of the unit is a token (r < L; on cut tilings also inside the grid).
  // Row 0 always is: the origin of a window, or offset p of the first window.
  auto present = [&](uint32_t r) -> bool {
    if constexpr (CUT) return r < L && cut_present(a, ud, r);
    return r < L;
  };

  // ---- prologue: the query rows go straight into the B-operand registers first, so
  // their latency overlaps the row tables
  bf16x8 qf[D / 16];
  {
    const uint32_t qrow = CUT ? (present(q0 + l32) ? q0 + l32 : 0) : min(q0 + l32, L - 1);
    const __bf16* qr = qg + row_elems<WIDE, D>(a.mqk.row_off(qrow)) + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(qr + kk * 16);
  }
  // units of at most TABLE_ROWS rows: every row's offset is formed once, into LDS
  __shared__ uint32_t ktab[TAB ? TABLE_ROWS : 1];
  __shared__ uint32_t vtab[TAB ? TABLE_ROWS : 1];
  // cut tilings: which rows are present, per 32-row key block and per lane half.
  // A lane of half h holds score registers r = 0..15 for the block's rows
  // 8*(r/4) + 4*h + r%4 (the MFMA output layout); entry 2*kb + h has bit r set
  // when that row is present, so the score mask tests constant bit positions.
  __shared__ uint32_t rmask[CUT && TAB ? TABLE_ROWS / 16 : 1];
  if constexpr (CUT && TAB) {
    // byte offsets; absent rows (and rows past the end, up to a whole block) read row 0
    const uint32_t iters = (nkb * BN + C::NT - 1) / C::NT;
    for (uint32_t i = 0; i < iters; ++i) {
      const uint32_t r = i * C::NT + tid;
      const bool ok = r < nkb * BN && present(r);
      const uint32_t rr = ok ? r : 0;
      const int32_t ko = a.mqk.row_off(rr);
      if (r < nkb * BN) {
        ktab[r] = bytes16(ko);
        vtab[r] = bytes16(a.v_like_k ? ko : a.mv.row_off(rr));
      }
      const uint64_t bits = __ballot(ok);
      // this wave's 64 rows are key blocks w0 and w0 + 1; lanes 0..3 each compact
      // one (block, half) pair: the nibbles at 4*h, 8 + 4*h, 16 + 4*h, 24 + 4*h
      const uint32_t w0 = (i * C::NT + 64 * wave) / 32;
      if (lane < 4 && w0 + (lane >> 1) < TABLE_ROWS / 32)
        rmask[2 * w0 + lane] = half_bits((uint32_t)(bits >> (32 * (lane >> 1))), lane & 1);
    }
  } else if constexpr (TAB) {
    // byte offsets; rows past the end of the unit (up to a whole block) repeat its last row
    for (uint32_t r = tid; r < nkb * BN; r += C::NT) {
      const uint32_t rr = min(r, L - 1);
      const int32_t ko = a.mqk.row_off(rr);
      ktab[r] = bytes16(ko);
      vtab[r] = bytes16(a.v_like_k ? ko : a.mv.row_off(rr));
    }
  }
  if constexpr (TAB) {
    // the table writes have completed; the barrier publishes them (no vmcnt wait:
    // the query rows may still be in flight)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }

  const bool v_like_k = a.v_like_k != 0;
  // cut tilings without the tables: this half's presence bits of the block in
  // each stage (formed when the block's loads are prepared)
  uint32_t kmask[3] = {0xffffu, 0xffffu, 0xffffu};

  // K: this wave's share of the block's direct loads.  Load `ins` fills rows
  // KRPI * ins ...; lane i carries row KRPI * ins + i / CPR, stored slot i % CPR,
  // i.e. chunk (i % CPR) ^ (row % CPR).
  const uint32_t krow0 = lane / C::CPR;
  const uint32_t kslot = lane % C::CPR;
  // direct loads this wave issues per block, for K and for V each
  const int my_loads = __builtin_amdgcn_readfirstlane((C::VINS - (int)wave + NW - 1) / NW);
  // wait until only this wave's loads of the newest block may be in flight
  auto wait_loads = [&](bool newest_in_flight) {
    if (!newest_in_flight) {
      wait_vmcnt<0>();
    } else if constexpr (C::VINS % NW == 0) {
      wait_vmcnt<2 * (C::VINS / NW)>();
    } else {
      wait_newest(my_loads);
    }
  };
  // V: load `ins` fills 4-row groups GPI * ins ...; lane i carries row
  // 4 * group + i % 4, chunk (i % (4 * CPR)) / 4.
  const uint32_t vrow0 = 4 * (lane / (4 * C::CPR)) + (lane & 3);
  const uint32_t vcol = (lane % (4 * C::CPR)) >> 2;
  // Loads of one block are prepared (row offsets located, lanes' 32-bit element
  // offsets formed) one step before they are issued, so the shuffles and the
  // address arithmetic stay off the path between a block's barrier and its MFMAs.
  boff_t pk[C::VPW], pv[C::VPW];
  auto prep_block = [&](uint32_t kb, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    if constexpr (TAB) {
#pragma unroll
      for (int i = 0; i < C::VPW; ++i) {
        const int ins = wave + i * NW;
        const uint32_t krow = C::KRPI * ins + krow0;
        const uint32_t kchunk = kslot ^ (krow & (C::CPR - 1));
        pk[i] = ktab[kb * BN + (krow & 31)] + kchunk * 16;
        pv[i] = vtab[kb * BN + ((4 * C::GPI * ins + vrow0) & 31)] + vcol * 16;
      }
    } else {
      // lane l (< 32) locates key l of the block; lanes 32-63 mirror lanes 0-31.
      // Rows past the end read the last row; on cut tilings absent rows read row 0
      uint32_t r = kb * BN + l32;
      if constexpr (CUT) {
        const bool ok = present(r);
        kmask[ST] = half_bits((uint32_t)__ballot(ok), half);
        r = ok ? r : 0;
      } else {
        r = min(r, L - 1);
      }
      const int32_t ko = a.mqk.row_off(r);
      const int32_t vo = v_like_k ? ko : a.mv.row_off(r);
#pragma unroll
      for (int i = 0; i < C::VPW; ++i) {
        const int ins = wave + i * NW;
        const uint32_t krow = C::KRPI * ins + krow0;
        const uint32_t kchunk = kslot ^ (krow & (C::CPR - 1));
        pk[i] = row_bytes16<WIDE, D>(shfl(ko, krow & 31)) + kchunk * 16;
        pv[i] = row_bytes16<WIDE, D>(shfl(vo, (4 * C::GPI * ins + vrow0) & 31)) + vcol * 16;
      }
    }
  };
  // the prepared block's K and V rows into stage ST
  auto issue_block = [&](auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    __bf16* ks = Stage<D, ST>::k();
    VT* vs = (VT*)Stage<D, ST>::v();
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const int ins = wave + i * NW;
      if (C::VPW * NW != C::VINS && ins >= C::VINS) break;
      // uniform base + unsigned 32-bit byte offset: one offset register per load
      // (wide maps: a 64-bit offset)
      __builtin_amdgcn_global_load_lds((const void*)((const char*)kg + pk[i]),
                                       (lds_void_t*)(ks + ins * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)((const char*)vg + pv[i]),
                                       (lds_void_t*)(vs + ins * 512), 16, 0, 0);
    }
  };

  // blocks 0 and 1 requested
  prep_block(0, std::integral_constant<int, 0>{});
  issue_block(std::integral_constant<int, 0>{});
  if (nkb > 1) {
    prep_block(1, std::integral_constant<int, 1>{});
    issue_block(std::integral_constant<int, 1>{});
  }
  if (nkb > 2) prep_block(2, std::integral_constant<int, 2>{});
  wait_vmcnt<0>();   // the query rows and blocks 0 and 1 have landed
  __builtin_amdgcn_s_barrier();

  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
  float m_ref = -INFINITY;   // reference max of the scaled logits (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum
  const float c = a.c;

  // transposing-read coordinates of V: lane l reads keys 4 * half + (l & 15) / 4
  // (+ 8 for the second read) at dims 16 * ((l >> 4) & 1) + 4 * (l & 3) of each
  // 32-dim tile, located in the chunk-interleaved groups
  const uint32_t tdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t toff = half * C::VGRP + 8 * (4 * (tdim >> 3) + ((lane & 15) >> 2)) + (tdim & 7);
  // the A operand of the scores: row l32, logical chunk 2 kk + half, stored at
  // slot (2 kk + half) ^ (l32 % CPR)
  const uint32_t kxor = l32 & (C::CPR - 1);
  // byte offset of this lane's K chunk 2 kk + half in any stage (row l32, swizzled slot)
  uint32_t kofs[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kofs[kk] = l32 * D * 2 + ((((uint32_t)(2 * kk) + half) ^ kxor) << 4);

  // one key block held in stage ST; requests block kb + 2 into stage (ST + 2) % 3.
  // ALL: blocks kb + 2 and kb + 3 exist (known at compile time, so the steps of the
  // main loop have no conditional loads and the compiler's waits stay exact)
  auto step = [&](uint32_t kb, auto st_tag, auto all_tag) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool ALL = decltype(all_tag)::value;
    const bool has2 = ALL || kb + 2 < nkb;
    // (the compiler waits for every outstanding load before the first LDS read after
    // the loop head, so in the loop's first step the loads go out after the scores)
    if (ST != 0 && has2) issue_block(std::integral_constant<int, (ST + 2) % 3>{});

    if (active) {
      const char* ks = (const char*)Stage<D, ST>::k();
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const char* kp = ks + kofs[kk];
        const uint2 lo = *(const uint2*)kp;
        const uint2 hi = *(const uint2*)(kp + 8);
        const bf16x8 kf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc, 0, 0, 0);
      }
      // the direct loads above read their offset registers after issue: keep those
      // registers from being reused as destinations of the reads just above
#pragma unroll
      for (int i = 0; i < C::VPW; ++i) asm volatile("" ::"v"(pk[i]), "v"(pv[i]));
      if (ST == 0 && has2) issue_block(std::integral_constant<int, (ST + 2) % 3>{});
      // keys past the end of the unit take no weight
      if constexpr (CUT) {
        uint32_t km;
        if constexpr (TAB) km = rmask[2 * kb + half];
        else km = kmask[ST];
        if (km != 0xffffu) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!__builtin_amdgcn_ubfe(km, r, 1)) sc[r] = -INFINITY;
        }
      } else if ((kb + 1) * BN > L) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t key = kb * BN + 8 * (r / 4) + 4 * half + (r % 4);
          if (key >= L) sc[r] = -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = max_halves(mx) * c;
      if (kb == 0) {
        m_ref = mx;
      } else if (__any(mx > m_ref + RESCALE_TAU)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha;
      }
      vx8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[r / 8][r % 8] = (VT)__builtin_amdgcn_exp2f(fmaf(sc[r], c, -m_ref));
      // the row sum adds the rounded weights the products use, two per instruction
      l_run = row_sum(pb, l_run);
      // O^T += V^T P^T, 16 keys per MFMA
      const VT* vs = (const VT*)Stage<D, ST>::v() + toff;
#pragma unroll
      for (int jk = 0; jk < 2; ++jk) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          // keys 16 jk + ... are groups 4 jk + half (+2); dims 32 mt + ... are chunks 4 mt + ...
          const VT* p1 = vs + 4 * jk * C::VGRP + 4 * 8 * 4 * mt;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(__attribute__((address_space(3))) VT*)p1);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(__attribute__((address_space(3))) VT*)(p1 + 2 * C::VGRP));
          const vx4 lo4 = __builtin_bit_cast(vx4, lo);
          const vx4 hi4 = __builtin_bit_cast(vx4, hi);
          vx8 va;
          va[0] = lo4[0]; va[1] = lo4[1]; va[2] = lo4[2]; va[3] = lo4[3];
          va[4] = hi4[0]; va[5] = hi4[1]; va[6] = hi4[2]; va[7] = hi4[3];
          acc[mt] = Vec<VT>::mfma(va, pb[jk], acc[mt]);
        }
      }
    }
    if (ST == 0 && has2 && !active) issue_block(std::integral_constant<int, (ST + 2) % 3>{});
    if (ALL || kb + 3 < nkb) prep_block(kb + 3, st_tag);
    // this wave's loads of block kb + 1 have landed (only block kb + 2 may be in
    // flight); the barrier then publishes them and retires stage ST's readers
    wait_loads(has2);
    __builtin_amdgcn_s_barrier();
  };
  // whole rounds of three steps (first those whose blocks all have successors to
  // request, then the last rounds), then the remainder: every path through a loop
  // body is the same, so the compiler can tell which stage's loads are in flight
  uint32_t kb = 0;
  for (; kb + 6 <= nkb; kb += 3) {
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

  // ---- epilogue: normalise; each wave stages its 32 rows in a free stage buffer
  // (chunk c of row r at slot c ^ (r % CPR)) and stores them as 16-byte chunks
  OT* ostage = (OT*)(wave == 0 ? Stage<D, 0>::k() : wave == 1 ? Stage<D, 1>::k()
                     : wave == 2 ? Stage<D, 2>::k() : Stage<D, 0>::v());
  if (NW > 4) ostage = nullptr;  // (only 2- and 4-wave workgroups are launched)
  if (active) {
    const float lsum = sum_halves(l_run);
    const float inv = 1.f / lsum;
    OT* orow = ostage + l32 * D + 4 * half;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ox4 w;
        w[0] = (OT)(acc[mt][4 * g + 0] * inv);
        w[1] = (OT)(acc[mt][4 * g + 1] * inv);
        w[2] = (OT)(acc[mt][4 * g + 2] * inv);
        w[3] = (OT)(acc[mt][4 * g + 3] * inv);
        *(ox4*)(orow + (((4 * mt + g) ^ kxor) << 3)) = w;
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the staged rows are in LDS
    __builtin_amdgcn_wave_barrier();
    constexpr int WR = 64 / C::CPR;   // rows per wave pass
    const uint32_t wcol = lane % C::CPR;
    const uint32_t wrow = lane / C::CPR;
    bool qok = q0 + l32 < L;
    if constexpr (CUT && TAB) {
      // row x of block x / 32 sits in half (x / 4) % 2 at register 4 * ((x % 32) / 8) + x % 4
      const uint32_t x = q0 + l32;
      qok = qok && ((rmask[2 * (x >> 5) + ((x >> 2) & 1)] >> (4 * ((x & 31) >> 3) + (x & 3))) & 1);
    } else if constexpr (CUT) {
      qok = qok && present(q0 + l32);
    }
    if (a.lse && qok && half == 0) a.lse[(size_t)u * L + q0 + l32] = m_ref + __log2f(lsum);
    const uint32_t oo = qok ? (uint32_t)a.mo.row_off(q0 + l32) : kNoRow;
#pragma unroll
    for (int i = 0; i < 32 / WR; ++i) {
      const uint32_t r = wrow + i * WR;
      const uint32_t o = (uint32_t)shfl((int)oo, r);
      const uint4 x = *(const uint4*)(ostage + r * D + ((wcol ^ (r & (C::CPR - 1))) << 3));
      if (o != kNoRow) *(uint4*)(og + row_elems<WIDE, D>((int32_t)o) + wcol * 8) = x;
    }
  }
}

template <int D, int NW, typename VT, typename OT, typename Args>
hipError_t launch(const Args& a, hipStream_t stream) {
  const uint32_t groups = (a.units + 7) / 8;
  const uint64_t blocks = (uint64_t)groups * 8 * a.nchunks;
  if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if constexpr (std::is_same<Args, AttnArgs>::value) {
    if (a.row_unit > 1) {
      // wide maps: no row tables, presence tested per block (the host marks every
      // wide call as cut; on a whole tiling every row is present)
      if (!a.cut.on) return hipErrorInvalidValue;
      hipLaunchKernelGGL((attn16_kernel<D, NW, VT, OT, false, true, AttnArgs, true>), dim3((uint32_t)blocks),
                         dim3(64 * NW), 0, stream, a);
      return hipGetLastError();
    }
    if (a.cut.on) {
      if (a.L <= TABLE_ROWS)
        hipLaunchKernelGGL((attn16_kernel<D, NW, VT, OT, true, true>), dim3((uint32_t)blocks), dim3(64 * NW), 0,
                           stream, a);
      else
        hipLaunchKernelGGL((attn16_kernel<D, NW, VT, OT, false, true>), dim3((uint32_t)blocks), dim3(64 * NW), 0,
                           stream, a);
      return hipGetLastError();
    }
  } else if (a.cut.on || a.row_unit > 1) {
    return hipErrorInvalidValue;
  }
  if (a.L <= TABLE_ROWS)
    hipLaunchKernelGGL((attn16_kernel<D, NW, VT, OT, true, false, Args>), dim3((uint32_t)blocks), dim3(64 * NW),
                       0, stream, a);
  else
    hipLaunchKernelGGL((attn16_kernel<D, NW, VT, OT, false, false, Args>), dim3((uint32_t)blocks), dim3(64 * NW),
                       0, stream, a);
  return hipGetLastError();
}

template <int D, typename VT, typename OT, typename Args>
hipError_t launch_nw(const Args& a, int nw, hipStream_t stream) {
  return nw == 4 ? launch<D, 4, VT, OT>(a, stream) : launch<D, 2, VT, OT>(a, stream);
}

template <typename VT, typename OT, typename Args>
hipError_t launch_types(const Args& a, int head_dim, int nw, hipStream_t stream) {
  if (head_dim == 128) return launch_nw<128, VT, OT>(a, nw, stream);
  if (head_dim == 64) return launch_nw<64, VT, OT>(a, nw, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// Waves per workgroup: 2 for units of at most 64 rows, else 4.  Measured on the
// high-resolution and 5B-DiT-shaped workloads, 4-wave workgroups (three per CU at
// this kernel's register and LDS use) beat 3-, 5-, 6- and 8-wave ones even where
// those leave fewer idle waves on a unit's last query chunk: more independent
// workgroups per CU hide the per-block barrier and load latency better.
int pick_waves(uint32_t L) { return L > 64 ? 4 : 2; }

hipError_t launch_attn_bf16(AttnArgs a, int head_dim, VType vtype, hipStream_t stream) {
  const uint32_t tiles = (a.L + 31) / 32;
  const int nw = pick_waves(a.L);
  a.nchunks = (tiles + nw - 1) / nw;
  switch (vtype) {
    case VType::kBf16ToBf16: return launch_types<__bf16, __bf16>(a, head_dim, nw, stream);
    case VType::kBf16ToF16: return launch_types<__bf16, _Float16>(a, head_dim, nw, stream);
    case VType::kF16ToBf16: return launch_types<_Float16, __bf16>(a, head_dim, nw, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16_k(AttnArgsK a, int head_dim, hipStream_t stream) {
  const uint32_t tiles = (a.L + 31) / 32;
  const int nw = pick_waves(a.L);
  a.nchunks = (tiles + nw - 1) / nw;
  return launch_types<_Float16, _Float16>(a, head_dim, nw, stream);
}

}  // namespace squad
