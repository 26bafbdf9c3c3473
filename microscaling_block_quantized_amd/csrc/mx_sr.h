// Stochastic rounding for the MX cast.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §4: the 4-bit pretraining recipe rounds
// gradients stochastically (and §8 lists stochastic rounding among the P3109
// rounding modes). The rule used here: a scaled value s with |s| < max moves to
// the grid value above |s| when the fraction f of |s| between its two
// neighbouring grid values exceeds u / 2^16 for a 16-bit random draw u, and to
// the one below otherwise; |s| >= max saturates and the sign is kept. The
// shared scale is chosen exactly as for round-to-nearest-even.
//
// The draws come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11) keyed by the caller's 64-bit
// seed: element i of X's flat [batch][rows][cols] order takes the low (i even)
// or high (i odd) 16 bits of word (i >> 1) & 3 of the block at counter
// (i >> 3, 0, 0). Both copies of an element (row and column) use its draw.
#pragma once
#include "mx_device.h"

namespace mx {

enum Round : int { kRne = 0, kSr = 1 };

// Ten rounds; each multiplies words 0 and 2 by the two Philox constants
// (32x32 -> 64-bit) and mixes the halves with words 1 and 3 and the key, which
// advances by the two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = uint64_t(0xD2511F53u) * c.x;
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c.z;
    c = make_uint4(uint32_t(p1 >> 32) ^ c.y ^ k0, uint32_t(p1), uint32_t(p0 >> 32) ^ c.w ^ k1, uint32_t(p0));
  }
  return c;
}

// Draws of the 8 elements 8g .. 8g+7.
__device__ __forceinline__ uint4 sr_words(uint64_t g, uint32_t seed_lo, uint32_t seed_hi) {
  return philox4x32_10(make_uint4(uint32_t(g), uint32_t(g >> 32), 0u, 0u), seed_lo, seed_hi);
}

// Grid of each element format: mantissa bits, smallest normal exponent and
// largest finite value (INT8 ignores the first two: its spacing is 2^-6).
template <int F> struct SrC;
template <> struct SrC<kE4M3> { static constexpr int mbits = 3, emin = -6; static constexpr float vmax = 448.0f; };
template <> struct SrC<kE5M2> { static constexpr int mbits = 2, emin = -14; static constexpr float vmax = 57344.0f; };
template <> struct SrC<kE2M1> { static constexpr int mbits = 1, emin = 0; static constexpr float vmax = 6.0f; };
template <> struct SrC<kE2M3> { static constexpr int mbits = 3, emin = 0; static constexpr float vmax = 7.5f; };
template <> struct SrC<kE3M2> { static constexpr int mbits = 2, emin = -2; static constexpr float vmax = 28.0f; };
template <> struct SrC<kInt8> { static constexpr int mbits = 6, emin = 0; static constexpr float vmax = 127.0f / 64.0f; };

// x (FP32 bits) divided by 2^e (e = scale code - 127) and rounded
// stochastically onto the element grid, returned as that grid value (exact in
// FP32: at most max and a multiple of the format's smallest spacing), which
// the nearest-even encoders given scale code 127 (2^0) map to its own code.
// |x| >= max * 2^e gives +-max. The fraction is compared as integers:
// |x| = M * 2^lsb, the grid spacing at |x| is 2^eq, and the d = eq - lsb low
// bits of M are the remainder, so the decision is exact for every FP32 input
// and no intermediate can overflow or underflow.
template <int F>
__device__ __forceinline__ float sr_scaled(uint32_t xb, int e, uint32_t u) {
  const uint32_t ab = xb & 0x7FFFFFFFu;
  const uint32_t sign = xb & 0x80000000u;
  const float lim = __builtin_ldexpf(SrC<F>::vmax, e);          // exact, or +Inf
  if (!(__uint_as_float(ab) < lim)) return __uint_as_float(sign | __float_as_uint(SrC<F>::vmax));
  if (ab == 0u) return __uint_as_float(xb);
  const uint32_t field = ab >> 23;
  const uint32_t mant = field ? ((ab & 0x7FFFFFu) | 0x800000u) : ab;
  const int lsb = (field ? int(field) : 1) - 150;
  int eq;
  if constexpr (F == kInt8) {
    eq = e - 6;
  } else {
    const int top = field ? int(field) - 127 : (31 - __builtin_clz(mant)) - 149;   // floor(log2 |x|)
    eq = max(top, e + SrC<F>::emin) - SrC<F>::mbits;
  }
  const int d = eq - lsb;                                      // bits of M below the spacing
  if (d <= 0) return __uint_as_float(sign | __float_as_uint(__builtin_ldexpf(__uint_as_float(ab), -e)));
  uint32_t n;
  bool up;
  if (d < 24) {
    n = mant >> d;
    up = (uint64_t(mant & ((1u << d) - 1u)) << 16) > (uint64_t(u) << d);
  } else {                                                     // |x| is below one spacing
    n = 0u;
    up = d >= 40 ? (u == 0u) : ((uint64_t(mant) << 16) > (uint64_t(u) << d));
  }
  // n + up <= 2^(mbits+1) (INT8: 127) and 2^(eq - e) >= 2^-16: exact
  const float v = float(n + (up ? 1u : 0u)) * __uint_as_float(uint32_t(eq - e + 127) << 23);
  return __uint_as_float(sign | __float_as_uint(v));
}

// sr_scaled without branches: |x| = M * 2^lsb and the grid spacing at |x| is
// 2^eq, so with d = eq - lsb the grid index below |x| is n = M >> d and the
// fraction is the d low bits of M. That fraction scaled by 2^32 is compared
// with u * 2^16: for d <= 32 it is M << (32 - d) exactly; for d > 32 it is
// M >> (d - 32) plus a sticky bit for the bits shifted out, which decides the
// tie. All 32-bit.
template <int F>
__device__ __forceinline__ float sr_scaled_flat(uint32_t xb, int e, uint32_t u) {
  const uint32_t ab = xb & 0x7FFFFFFFu;
  const uint32_t sign = xb & 0x80000000u;
  const float lim = __builtin_ldexpf(SrC<F>::vmax, e);          // exact, or +Inf
  const uint32_t field = ab >> 23;
  const uint32_t mant = field ? ((ab & 0x7FFFFFu) | 0x800000u) : ab;
  const int lsb = (field ? int(field) : 1) - 150;
  int eq;
  if constexpr (F == kInt8) {
    eq = e - 6;
  } else {
    const int top = field ? int(field) - 127 : (31 - __builtin_clz(mant | 1u)) - 149;   // floor(log2 |x|)
    eq = max(top, e + SrC<F>::emin) - SrC<F>::mbits;
  }
  const int d = eq - lsb;
  const uint32_t n = d <= 0 ? mant << uint32_t(min(-d, 31)) : (d >= 32 ? 0u : mant >> uint32_t(d));
  const uint32_t sh = uint32_t(min(max(d - 32, 0), 24));
  const uint32_t rem = d <= 32 ? mant << uint32_t(min(max(32 - d, 0), 31)) : mant >> sh;
  const bool lost = d > 32 && (mant & ((1u << sh) - 1u)) != 0u;
  const uint32_t thr = u << 16;
  const bool up = d >= 1 && (rem > thr || (rem == thr && lost));
  const float v = float(n + (up ? 1u : 0u)) * __uint_as_float(uint32_t(eq - e + 127) << 23);
  uint32_t r = ab == 0u ? xb : (sign | __float_as_uint(v));
  r = __uint_as_float(ab) < lim ? r : (sign | __float_as_uint(SrC<F>::vmax));
  return __uint_as_float(r);
}

// The same decision through the FP32 pipeline, for every input but FP32
// subnormals and the tiniest elements of a block. With eq the exponent of the
// grid spacing at |x| (as above), y = |x| / 2^eq is exact while it is a normal
// number, and so are n = floor(y) and the fraction y - n. The rule "fraction
// > u / 2^16" is then the exact comparison fraction * 2^16 > u, both sides
// exact in FP32, and (n or n + 1) * 2^(eq - e) is the exact grid value. Sets
// `slow` for an FP32-subnormal x (whose exponent field does not give
// floor(log2 |x|)) and for a y below 2^-126. The caller then recomputes with
// sr_scaled_flat. Zero needs no case of its own: y = 0 never rounds up.
template <int F>
__device__ __forceinline__ float sr_scaled_fast(uint32_t xb, int e, float lim, uint32_t u, bool& slow) {
  const uint32_t ab = xb & 0x7FFFFFFFu;
  const int field = int(ab >> 23);
  int eq;
  if constexpr (F == kInt8) eq = e - 6;
  else eq = max(field - 127, e + SrC<F>::emin) - SrC<F>::mbits;
  const float y = __builtin_ldexpf(__uint_as_float(ab), -eq);
  const float n = __builtin_floorf(y);
  const bool up = (y - n) * 65536.0f > float(u);
  const float v = __builtin_ldexpf(up ? n + 1.0f : n, eq - e);
  slow |= (field == 0 || y < 0x1p-126f) && ab != 0u;
  const bool sat = !(__uint_as_float(ab) < lim);
  const uint32_t mag = sat ? __float_as_uint(SrC<F>::vmax) : __float_as_uint(v);
  return __uint_as_float((xb & 0x80000000u) | mag);
}

// N elements. FAST: through the fast path, redone with sr_scaled_flat when any
// lane of the wave needs it (one branch per group). Otherwise sr_scaled per
// element, which needs the fewest registers (the FP32 row+column kernel).
template <int F, int N, bool FAST>
__device__ __forceinline__ void sr_scaled_n(const uint32_t* xb, int e, const uint32_t* u, float* f) {
  if constexpr (FAST) {
    const float lim = __builtin_ldexpf(SrC<F>::vmax, e);
    bool slow = false;
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = sr_scaled_fast<F>(xb[i], e, lim, u[i], slow);
    if (slow) {
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] = sr_scaled_flat<F>(xb[i], e, u[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = sr_scaled<F>(xb[i], e, u[i]);
  }
}

// Scale code for encoding values that sr_scaled already divided by 2^e: 2^0,
// or the NaN code that makes the encoders write a NaN block.
__device__ __forceinline__ uint32_t sr_enc_code(uint32_t code) { return code == 0xFFu ? 0xFFu : 127u; }

// Stochastic-rounding encoders on top of the nearest-even ones: each element
// is first moved onto the grid (sr_scaled), which the nearest-even encoder then
// maps to its own code. Output layout as encode8_bf16 (BF16: 8 elements) or
// encode4_f32 (FP32: 4 elements, in .x).
template <bool BF16, int F, int M, bool FAST>
__device__ __forceinline__ uint2 encode8_sr(const uint4& v, const uint32_t* draw, uint32_t code) {
  const int e = int(code) - 127;
  const uint32_t ec = sr_enc_code(code);
  if constexpr (BF16) {
    float f[8];
    uint32_t xb[8], uu[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = (&v.x)[i];
      xb[2 * i] = p << 16;
      xb[2 * i + 1] = p & 0xFFFF0000u;
      uu[2 * i] = draw[i] & 0xFFFFu;
      uu[2 * i + 1] = draw[i] >> 16;
    }
    sr_scaled_n<F, 8, FAST>(xb, e, uu, f);
    const uint32_t lo = encode4_f32<F, M>(f[0], f[1], f[2], f[3], ec);
    const uint32_t hi = encode4_f32<F, M>(f[4], f[5], f[6], f[7], ec);
    if constexpr (F == kE2M1) return make_uint2((lo & 0xFFFFu) | (hi << 16), 0u);
    else return make_uint2(lo, hi);
  } else {
    float f[4];
    uint32_t uu[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) uu[i] = (i & 1) ? (draw[i >> 1] >> 16) : (draw[i >> 1] & 0xFFFFu);
    sr_scaled_n<F, 4, FAST>(&v.x, e, uu, f);
    return make_uint2(encode4_f32<F, M>(f[0], f[1], f[2], f[3], ec), 0u);
  }
}

// One column of 8 BF16 rows (pairs pr[i] = rows 2i (low half) and 2i+1) with
// the rows' draws dj[0..7].
template <int F, int M, bool FAST>
__device__ __forceinline__ uint2 encode_col_sr(const uint32_t* pr, const uint32_t* dj, uint32_t code) {
  const int e = int(code) - 127;
  const uint32_t ec = sr_enc_code(code);
  float f[8];
  uint32_t xb[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xb[2 * i] = pr[i] << 16;
    xb[2 * i + 1] = pr[i] & 0xFFFF0000u;
  }
  sr_scaled_n<F, 8, FAST>(xb, e, dj, f);
  const uint32_t lo = encode4_f32<F, M>(f[0], f[1], f[2], f[3], ec);
  const uint32_t hi = encode4_f32<F, M>(f[4], f[5], f[6], f[7], ec);
  if constexpr (F == kE2M1) return make_uint2((lo & 0xFFFFu) | (hi << 16), 0u);
  else return make_uint2(lo, hi);
}

}  // namespace mx
