// squad_kernels.h - launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "squad_map.h"

namespace squad {

// One launch runs `units` independent softmax attentions of L rows each: for unit u
// and query row i, out_i = sum_j softmax_j(scale * <q_i, k_j>) v_j over the unit's L
// rows.  Units are numbered u = s * BH + bh (s = unit within a (batch, head) pair,
// bh = batch * heads + head), so neighbouring units are the heads of one window or
// group.  Rows of q and k are located with mqk, rows of v with mv, output rows
// with mo.
// Tilings cut by the grid edge: a grid that is not a whole number of tiles is
// padded up to one with absent tokens.  Row r of unit s is present iff, on every
// axis (t, h, w), unit digit * su + row digit * sr < lim, where the digits are
// those of the token map (unit: window or offset digits, row: the other kind).
struct Cut {
  uint32_t on;       // nonzero: some rows are absent
  uint32_t lim[3];   // T, H, W
  uint32_t su[3];    // per-axis scale of the unit's digit
  uint32_t sr[3];    // per-axis scale of the row's digit
};

template <typename Map>
struct AttnArgsT {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  Map mqk, mv, mo;
  uint32_t L;        // rows (queries = keys) per unit
  uint32_t U;        // units per (batch, head)
  uint32_t heads;    // heads per batch element
  uint32_t BH;       // batch * heads
  FastDiv fBH, fHeads;
  uint32_t units;    // BH * U
  uint32_t nchunks;  // query chunks per unit (set by the launcher)
  uint32_t v_like_k; // nonzero: mv locates rows exactly as mqk does
  float c;           // softmax scale * log2(e)
  Cut cut;           // absent rows (cut tilings only; on == 0 otherwise)
  float* lse;        // optional: row statistics lse[u * L + r] = log2 sum_j exp2(c <q_r, k_j>)
  uint32_t row_unit; // elements per unit of the maps' row offsets: 1 (narrow), head_dim (wide)
};
typedef AttnArgsT<RowMap> AttnArgs;
typedef AttnArgsT<RowMapK> AttnArgsK;   // six-digit units (middle passes of k levels)

// The digits of unit s under the token map, for Cut tests of its rows.
struct UnitDigits {
  uint32_t d[3];
};
template <typename Args>
__host__ __device__ __forceinline__ UnitDigits cut_unit_digits(const Args& a, uint32_t s) {
  UnitDigits u;
  a.mqk.unit.digits(s, u.d[0], u.d[1], u.d[2]);
  return u;
}
// Whether row r (< L) of the unit is a token of the grid.
template <typename Args>
__host__ __device__ __forceinline__ bool cut_present(const Args& a, const UnitDigits& u, uint32_t r) {
  uint32_t r2, r1, r0;
  a.mqk.row.digits(r, r2, r1, r0);
  return u.d[0] * a.cut.su[0] + r2 * a.cut.sr[0] < a.cut.lim[0] &&
         u.d[1] * a.cut.su[1] + r1 * a.cut.sr[1] < a.cut.lim[1] &&
         u.d[2] * a.cut.su[2] + r0 * a.cut.sr[2] < a.cut.lim[2];
}

// Value and output types of the bf16 engine (q and k are always bf16).  The local
// pass of squad_attn_forward writes its output as fp16 (three more significand bits
// than bf16, same bytes) and the global pass reads it back as fp16 values.
enum class VType { kBf16ToBf16, kBf16ToF16, kF16ToBf16 };

hipError_t launch_attn_bf16(AttnArgs a, int head_dim, VType vtype, hipStream_t stream);
hipError_t launch_attn_f32(AttnArgs a, int head_dim, hipStream_t stream);
// middle passes of a k-level operator: fp16 values in, fp16 out (bf16 calls)
hipError_t launch_attn_bf16_k(AttnArgsK a, int head_dim, hipStream_t stream);
hipError_t launch_attn_f32_k(AttnArgsK a, int head_dim, hipStream_t stream);

// Backward of one pass (the gradients of the unit attentions above), in two
// launches over the same units and rows:
//   kind A (per query row i):  D_i = <dout_i, o_i>;  dq_i = scale * sum_j dS_ij k_j
//   kind B (per key row j):    dv_j = sum_i P_ij dout_i;  dk_j = scale * sum_i dS_ij q_i
// with P_ij = exp2(c <q_i, k_j> - lse_i) and dS_ij = P_ij (<dout_i, v_j> - D_i).
// Kind A writes D (dsum) for kind B.  dq and dk are summed over the passes: with
// k levels, the first pass writes its part to fp32 accumulators (token order, the
// offsets of mdq / mdk), middle passes add to them, and the last adds them and
// writes dq / dk in the call's dtype (for fp32 calls the accumulators are dq and dk
// themselves).  The two-pass bf16 backward hands the global pass's dq and dk parts to the local
// pass in the dq and dk buffers themselves, as fp16 rows scaled by a power of two
// per row (the scale's inverse in dq_sc / dk_sc): kPartWrite writes them, kPartAdd
// (middle levels of k levels) adds to them, kPartFinal adds them and writes the
// bf16 gradients.
enum BwdAcc : uint32_t { kAccWrite = 0, kAccFinal = 1, kAccAdd = 2, kPartWrite = 3, kPartFinal = 4,
                         kPartAdd = 5 };
template <typename Map>
struct BwdArgsT {
  const void* q;
  const void* k;
  const void* v;      // value rows (the global pass: the local output)
  const void* o;      // this pass's output rows (kind A, for D)
  const void* dout;   // upstream gradient of this pass's output
  Map mqk, mv, mo, mdo;
  const float* lse;   // [u * L + r]
  float* dsum;        // [u * L + r]: D, written by kind A, read by kind B
  uint32_t dsum_ready;  // nonzero: dsum already holds D (kind A reads it instead of forming it)
  // optional (kind B, two-pass global pass): D of the pass below for this pass's
  // value rows, <dv_j, v_j>, at [(row * BH + bh) * U + unit] (the lower pass's
  // units are this pass's rows and its rows this pass's units)
  float* dsum_next;
  void* dq;           // kind A, final pass: dq in the call's dtype (token order, mdq)
  void* dk;           // kind B, final pass: dk
  float* dq_acc;      // fp32 accumulators (mdq / mdk offsets)
  float* dk_acc;
  float* dq_sc;       // kPart modes: per head row of dq / dk, the inverse scale of its part
  float* dk_sc;       // (index: the row's element offset / head_dim)
  void* dv;           // kind B: value gradient rows (mdv)
  Map mdq, mdk, mdv;
  uint32_t final_pass;  // BwdAcc mode of the dq and dk stores
  uint32_t L, U, heads, BH;
  FastDiv fBH, fHeads;
  uint32_t units, nchunks;
  float c;            // softmax scale * log2(e)
  float scale;
  Cut cut;
  uint32_t row_unit;  // elements per unit of the maps' row offsets: 1 (narrow), head_dim (wide)
};
typedef BwdArgsT<RowMap> BwdArgs;
typedef BwdArgsT<RowMapK> BwdArgsK;   // middle levels of a k-level operator

// Element types of the bf16 engine's backward launches (q, k, dout and the
// gradients are bf16; o and v may be the fp16 local output).
struct BwdTypes {
  bool v_f16;         // value rows are fp16 (the global pass: the local output)
  bool o_f16;         // output rows are fp16 (the local pass: the local output)
};

hipError_t launch_bwd_f32(BwdArgs a, int head_dim, bool kind_b, hipStream_t stream);
hipError_t launch_bwd_f32_k(BwdArgsK a, int head_dim, bool kind_b, hipStream_t stream);

// The measuring kernel: blocks x 256 threads, each wave `iters` rounds of four
// independent 32x32x16 bf16 MFMAs; out[blocks * 256] receives a checksum per lane.
hipError_t launch_mfma_probe(float* out, int32_t blocks, int32_t iters, hipStream_t stream);
hipError_t launch_bwd_bf16(BwdArgs a, int head_dim, BwdTypes t, bool kind_b, hipStream_t stream);
// middle levels: fp16 values and outputs
hipError_t launch_bwd_bf16_k(BwdArgsK a, int head_dim, bool kind_b, hipStream_t stream);
// Units of at most 64 rows on a whole tiling: one kernel forms dq, dk and dv
// (and D) in place of the two kinds.
bool bwd_bf16_fused(uint32_t L, bool cut);
hipError_t launch_bwd_bf16_small(BwdArgs a, int head_dim, BwdTypes t, hipStream_t stream);
hipError_t launch_bwd_bf16_small_k(BwdArgsK a, int head_dim, hipStream_t stream);

// Row-permutation copy: rows e = (bh * U + s) * L + r for bh < BH, s < U, r < L;
// row e is read at src + ms(b, h, s, r) and written at dst + md(b, h, s, r).
struct CopyArgs {
  const void* src;
  void* dst;
  RowMap ms, md;      // offsets in elements (rows: in units of row_unit elements)
  uint32_t L, U, heads, BH;
  FastDiv fL, fU, fHeads;
  uint32_t rows;      // BH * U * L
  uint32_t row_chunks_log2;  // log2 of the 16-byte chunks per row
  uint32_t elem_bytes;  // 2 or 4
  uint32_t row_unit;  // 1 (narrow maps) or head_dim (wide maps)
};

hipError_t launch_row_copy(CopyArgs a, hipStream_t stream);

}  // namespace squad
