// squad_map.h - address maps from (batch, head, unit, row) to tensor element offsets.
//
// Both passes of SQuad-Attention run one softmax attention per "unit": a window
// (local pass) or an offset group (global pass).  A unit's rows are its tokens.
// The maps below turn (b, h, unit s, row r) into the element offset of that row in
// a tensor, so the attention kernels read token-order inputs and write their
// outputs in place, with the window gather, the window-to-group regroup and the
// final scatter folded into their loads and stores.
//
// Every map has the form
//     off = b*sB + h*sH + mix(s; U1, U0; A2, A1, A0) + mix(r; R1, R0; C2, C1, C0)
// where mix(x; X1, X0; S2, S1, S0) splits x into mixed-radix digits
// (x2, x1, x0) with x0 = x % X0, x1 = (x / X0) % X1, x2 = x / (X0*X1) and returns
// x2*S2 + x1*S1 + x0*S0.  A token (t, h, w) of a T x H x W grid lies at token index
// (t*H + h)*W + w; with tile (tt, th, tw) and window grid (nt, nh, nw) =
// (T/tt, H/th, W/tw), window g = (gt*nh + gh)*nw + gw and offset
// p = (at*th + ah)*tw + aw sit at t = gt*tt + at, h = gh*th + ah, w = gw*tw + aw,
// so the token index splits into a window part and an offset part, each a
// mixed-radix mix of its digits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace squad {

// Division by a runtime constant d >= 1 for dividends x < 2^32:
// q = floor(x * M / 2^64) with M = ceil(2^64 / d) is exact because the error term
// x * (M*d - 2^64) / (d * 2^64) < x / 2^64 < 1/d (Granlund & Montgomery, 1994).
struct FastDiv {
  uint64_t mul;   // ceil(2^64 / d); unused for d == 1
  uint32_t d;

  __host__ __device__ FastDiv() : mul(0), d(1) {}
  __host__ explicit FastDiv(uint32_t divisor) : mul(0), d(divisor) {
    if (d > 1) {
      unsigned __int128 one = 1;
      mul = (uint64_t)(((one << 64) + d - 1) / d);
    }
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t x) const {
    if (d == 1) return x;
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)__umul64hi((uint64_t)x, mul);
#else
    return (uint32_t)(((unsigned __int128)x * mul) >> 64);
#endif
  }
};

// Division by a runtime constant d >= 1 for dividends x < 2^31 with one 32-bit
// high multiply: with l = ceil(log2 d), m = ceil(2^(31+l) / d) < 2^32 and
// q = floor(x * m / 2^(31+l)) is exact because x * (m*d - 2^(31+l)) < 2^31 * d
// <= 2^(31+l) (the same round-up method, for 31-bit dividends).
// d == 1 is folded in without a branch: mul = 0, pass = all ones, shift = 0.
struct FastDiv32 {
  uint32_t mul;    // ceil(2^(31+l) / d)
  uint32_t pass;   // ~0u for d == 1, else 0
  uint32_t shift;  // l - 1
  uint32_t d;

  __host__ __device__ FastDiv32() : mul(0), pass(~0u), shift(0), d(1) {}
  __host__ explicit FastDiv32(uint32_t divisor) : mul(0), pass(~0u), shift(0), d(divisor) {
    if (d > 1) {
      uint32_t l = 0;
      while ((uint64_t(1) << l) < d) ++l;
      mul = (uint32_t)(((uint64_t(1) << (31 + l)) + d - 1) / d);
      shift = l - 1;
      pass = 0;
    }
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t x) const {
#if defined(__HIP_DEVICE_COMPILE__)
    return (__umulhi(x, mul) + (x & pass)) >> shift;
#else
    return ((uint32_t)(((uint64_t)x * mul) >> 32) + (x & pass)) >> shift;
#endif
  }
};

// Unit part of a map: evaluated once per workgroup, 64-bit strides.
struct Mix {
  FastDiv x1, x0;     // radices X1, X0
  int64_t s2, s1, s0; // strides of the digits (elements)

  __host__ __device__ __forceinline__ int64_t at(uint32_t x) const {
    uint32_t q0 = x0.div(x);
    uint32_t d0 = x - q0 * x0.d;
    uint32_t q1 = x1.div(q0);
    uint32_t d1 = q0 - q1 * x1.d;
    return (int64_t)q1 * s2 + (int64_t)d1 * s1 + (int64_t)d0 * s0;
  }
  // the digits (x2, x1, x0) of x
  __host__ __device__ __forceinline__ void digits(uint32_t x, uint32_t& x2, uint32_t& x1d, uint32_t& x0d) const {
    const uint32_t q0 = x0.div(x);
    x0d = x - q0 * x0.d;
    x2 = x1.div(q0);
    x1d = q0 - x2 * x1.d;
  }
};

// Row part of a map: evaluated per key block in the attention loop, 32-bit (the
// host guarantees every row offset inside one (batch, head) is below 2^31 elements,
// or, for wide maps, below 2^32 - 1 head rows; see kNoRow).
struct Mix32 {
  FastDiv32 x1, x0;
  int32_t s2, s1, s0;

  __host__ __device__ __forceinline__ int32_t at(uint32_t x) const {
    uint32_t q0 = x0.div(x);
    uint32_t d0 = x - q0 * x0.d;
    uint32_t q1 = x1.div(q0);
    uint32_t d1 = q0 - q1 * x1.d;
    return (int32_t)(q1 * (uint32_t)s2 + d1 * (uint32_t)s1 + d0 * (uint32_t)s0);
  }
  __host__ __device__ __forceinline__ void digits(uint32_t x, uint32_t& x2, uint32_t& x1d, uint32_t& x0d) const {
    const uint32_t q0 = x0.div(x);
    x0d = x - q0 * x0.d;
    x2 = x1.div(q0);
    x1d = q0 - x2 * x1.d;
  }
};

// Byte offset of a 16-bit element at element offset e (0 <= e < 2^31) inside one
// (batch, head).  Formed in unsigned 32-bit arithmetic: exact up to 2^32 - 2 bytes
// and zero-extended where it is added to a pointer (doubling a signed offset would
// turn offsets of 2^30 elements and more negative).
__host__ __device__ __forceinline__ uint32_t bytes16(int32_t e) { return 2u * (uint32_t)e; }

// Narrow and wide row maps.  A narrow map (the default) holds row offsets in
// elements, below 2^31.  A wide map holds them in units of one head row (head_dim
// elements: every row stride of every map is a multiple of head_dim), below
// 2^32 - 1, for tensors whose rows inside one batch element span 2^31 elements
// or more (up to 2^32 - 1 head rows).  The unit part of a map is in elements either
// way (64-bit).  The all-ones offset never occurs, so it can mark an absent row.
constexpr uint32_t kNoRow = 0xffffffffu;

// Element offset of a row of a map with D-element head rows (narrow: the offset
// itself, non-negative, so it is added zero-extended).
template <bool WIDE, int D>
__host__ __device__ __forceinline__ typename std::conditional<WIDE, uint64_t, uint32_t>::type row_elems(int32_t e) {
  if constexpr (WIDE) return (uint64_t)(uint32_t)e * (uint64_t)D;
  else return (uint32_t)e;
}
// Byte offset of a row of a 16-bit tensor: narrow maps give an unsigned 32-bit
// offset (exact below 2^32 bytes; added zero-extended, so that the loads keep a
// uniform 64-bit base and one 32-bit offset register), wide maps a 64-bit one.
template <bool WIDE, int D>
__host__ __device__ __forceinline__ typename std::conditional<WIDE, uint64_t, uint32_t>::type row_bytes16(int32_t e) {
  if constexpr (WIDE) return (uint64_t)(uint32_t)e * (uint64_t)(2 * D);
  else return bytes16(e);
}
// The same at run time (engines whose kernels are not specialised on the width):
// `unit` is 1 for narrow maps and head_dim for wide ones.
__host__ __device__ __forceinline__ uint64_t row_elems_rt(int32_t e, uint32_t unit) {
  return (uint64_t)(uint32_t)e * unit;
}

struct RowMap {
  int64_t sB, sH; // batch and head strides (elements)
  Mix unit;       // unit index -> offset
  Mix32 row;      // row index  -> offset from the unit's base

  __host__ __device__ __forceinline__ int64_t base(uint32_t b, uint32_t h, uint32_t s) const {
    return (int64_t)b * sB + (int64_t)h * sH + unit.at(s);
  }
  __host__ __device__ __forceinline__ int32_t row_off(uint32_t r) const { return row.at(r); }
};

// A map whose unit index has six digits: s = hi * split + lo, lo and hi each a
// three-digit mix.  The middle passes of a k-level tiling need it: their units
// are (position inside the level-j tile, index of the level-(j+1) tile).
struct RowMapK {
  int64_t sB, sH;
  Mix unit;       // lo = s % split -> offset
  Mix outer;      // hi = s / split -> offset
  FastDiv split;
  Mix32 row;

  __host__ __device__ __forceinline__ int64_t base(uint32_t b, uint32_t h, uint32_t s) const {
    const uint32_t hi = split.div(s);
    return (int64_t)b * sB + (int64_t)h * sH + unit.at(s - hi * split.d) + outer.at(hi);
  }
  __host__ __device__ __forceinline__ int32_t row_off(uint32_t r) const { return row.at(r); }
};

}  // namespace squad
