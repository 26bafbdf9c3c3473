// MX dequantization: codes + E8M0 scales -> FP32 or BF16.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §7: an E8M0 scale is a power of two, so
// applying it is an exponent add with no rounding; §2: scale code 0xFF is NaN
// and turns all 32 elements of its block NaN. Each value is formed exactly as
// an FP32 (every element value times 2^(k-127) is an FP32 number, subnormals
// included) by the gfx950 scaled up-conversion, and BF16 output is that FP32
// rounded to nearest-even. NaN is written as the positive quiet NaN.
//
// E2M3 / E3M2 codes are decoded as their FP8 carrier (E4M3 / E5M2, the same
// values 2^6 / 2^12 lower, see mx_device.h) and multiplied back up, exactly.
// INT8 code k is the value (k ^ 0x80) - 128 in units of 2^(scale - 133).
//
// One thread handles 16 consecutive elements (half a block): a 16-byte (FP8,
// INT8), 12-byte (FP6) or 8-byte (E2M1) code load, one scale byte, and 64 or
// 32 bytes of output.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kDeqThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Codes are read with non-temporal loads; the outputs use ordinary stores
// (non-temporal stores made this write-heavy kernel 40% slower on MI355X).
__device__ __forceinline__ void store16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<u32x4*>(p) = u32x4{a, b, c, d};
}

__device__ __forceinline__ uint32_t canon_nan_f32(uint32_t b) {
  return (b & 0x7FFFFFFFu) > 0x7F800000u ? 0x7FC00000u : b;
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  // compiles to v_cvt_pk_bf16_f32 (round to nearest-even)
  const bf16x2 h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// Two FP8 codes (lo or hi half of c) times the scale, in element order.
template <int F>
__device__ __forceinline__ float2v fp8_pair(uint32_t c, float sc, bool hi) {
  if constexpr (F == kE4M3) return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, sc, true)
                                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, sc, false);
  else return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(c, sc, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(c, sc, false);
}

template <int F>
__device__ __forceinline__ void decode16(const uint32_t* cw, uint32_t k, float* o) {
  const float sc = scale_operand(k);
  if constexpr (kIsFp6<F>) {
    // 12 bytes -> four 24-bit groups of 4 codes -> carrier bytes (sign from bit 5 to bit 7)
    constexpr int CF = FmtC<F>::carrier;
    const float up = __uint_as_float(uint32_t(127 + FmtC<F>::shift) << 23);
    const uint32_t g[4] = {cw[0], (cw[0] >> 24) | (cw[1] << 8), (cw[1] >> 16) | (cw[2] << 16), cw[2] >> 8};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t c6 = unpack6(g[d]);
      const uint32_t c8 = (c6 & 0x1F1F1F1Fu) | ((c6 & 0x20202020u) << 2);
      const float2v lo = fp8_pair<CF>(c8, sc, false), hi = fp8_pair<CF>(c8, sc, true);
      o[4 * d + 0] = lo.x * up; o[4 * d + 1] = lo.y * up; o[4 * d + 2] = hi.x * up; o[4 * d + 3] = hi.y * up;
    }
  } else if constexpr (F == kInt8) {
    // unit 2^(k-133): an FP32 normal for k >= 7, else the subnormal with bit k+16 set;
    // the integer (exact in FP32) times the unit is exact, or overflows only when
    // the value itself does
    const float unit = __uint_as_float(k >= 7u ? (k - 6u) << 23 : 1u << (k + 16u));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t u = cw[d] ^ 0x80808080u;          // offset binary: byte = k + 128
#pragma unroll
      for (int b = 0; b < 4; ++b) o[4 * d + b] = (float((u >> (8 * b)) & 0xFFu) - 128.0f) * unit;
    }
  } else if constexpr (F == kE2M1) {
    // two dwords hold 16 codes, element 2k in the low nibble of byte k
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      float2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], sc, 0);
      float2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], sc, 1);
      float2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], sc, 2);
      float2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], sc, 3);
      o[8 * d + 0] = p0.x; o[8 * d + 1] = p0.y; o[8 * d + 2] = p1.x; o[8 * d + 3] = p1.y;
      o[8 * d + 4] = p2.x; o[8 * d + 5] = p2.y; o[8 * d + 6] = p3.x; o[8 * d + 7] = p3.y;
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float2v lo = fp8_pair<F>(cw[d], sc, false), hi = fp8_pair<F>(cw[d], sc, true);
      o[4 * d + 0] = lo.x; o[4 * d + 1] = lo.y; o[4 * d + 2] = hi.x; o[4 * d + 3] = hi.y;
    }
  }
}

// B2: 32x32 blocks over rows of `cols` elements; the scale of chunk i (row
// r = 16 i / cols, column c = 16 i % cols) is scales[(r / 32) * (cols / 32) + c / 32].
template <int F, bool OUT_BF16, bool B2>
__global__ __launch_bounds__(kDeqThreads) void mx_dequant_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             void* __restrict__ y, int64_t nchunks, int64_t cols) {
  const int64_t i = int64_t(blockIdx.x) * kDeqThreads + threadIdx.x;   // 16-element chunk
  if (i >= nchunks) return;
  int64_t si = i >> 1;
  if constexpr (B2) {
    const int64_t cpr = cols / 16;                                    // chunks per row
    const int64_t r = i / cpr, c = i - r * cpr;
    si = (r >> 5) * (cols >> 5) + (c >> 1);
  }
  const uint32_t k = scales[si];
  uint32_t cw[4];
  if constexpr (F == kE2M1) {
    const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + i * 8));
    cw[0] = c.x; cw[1] = c.y; cw[2] = 0; cw[3] = 0;
  } else if constexpr (kIsFp6<F>) {
    // three dword loads of consecutive addresses, merged into one 12-byte load
    const uint32_t* q = reinterpret_cast<const uint32_t*>(codes + i * 12);
    cw[0] = __builtin_nontemporal_load(q);
    cw[1] = __builtin_nontemporal_load(q + 1);
    cw[2] = __builtin_nontemporal_load(q + 2);
    cw[3] = 0;
  } else {
    const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + i * 16));
    cw[0] = c.x; cw[1] = c.y; cw[2] = c.z; cw[3] = c.w;
  }
  float o[16];
  decode16<F>(cw, k, o);
  uint32_t ob[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    ob[e] = k == 0xFFu ? 0x7FC00000u : canon_nan_f32(__float_as_uint(o[e]));
  if constexpr (OUT_BF16) {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t p = f32x2_to_bf16x2(__uint_as_float(ob[2 * e]), __uint_as_float(ob[2 * e + 1]));
      // keep the canonical NaN exact through the narrowing
      const bool n0 = (ob[2 * e] == 0x7FC00000u), n1 = (ob[2 * e + 1] == 0x7FC00000u);
      p = n0 ? ((p & 0xFFFF0000u) | 0x7FC0u) : p;
      p = n1 ? ((p & 0x0000FFFFu) | 0x7FC00000u) : p;
      h[e] = p;
    }
    uint8_t* dst = reinterpret_cast<uint8_t*>(y) + i * 32;
    store16(dst, h[0], h[1], h[2], h[3]);
    store16(dst + 16, h[4], h[5], h[6], h[7]);
  } else {
    uint8_t* dst = reinterpret_cast<uint8_t*>(y) + i * 64;
#pragma unroll
    for (int e = 0; e < 4; ++e) store16(dst + 16 * e, ob[4 * e], ob[4 * e + 1], ob[4 * e + 2], ob[4 * e + 3]);
  }
}

template <int F, bool B, bool B2>
hipError_t launch_dq(const uint8_t* c, const uint8_t* s, void* y, int64_t n, int64_t cols, hipStream_t st) {
  const int64_t chunks = n / 16;
  const int64_t blocks = (chunks + kDeqThreads - 1) / kDeqThreads;
  return launch_kernel(mx_dequant_kernel<F, B, B2>, dim3(uint32_t(blocks)), dim3(kDeqThreads), st, c, s, y, chunks,
                       cols);
}

template <int F>
hipError_t by_out(bool out_bf16, const uint8_t* c, const uint8_t* s, void* y, int64_t n, int64_t cols,
                  hipStream_t st) {
  if (cols > 0)
    return out_bf16 ? launch_dq<F, true, true>(c, s, y, n, cols, st) : launch_dq<F, false, true>(c, s, y, n, cols, st);
  return out_bf16 ? launch_dq<F, true, false>(c, s, y, n, 0, st) : launch_dq<F, false, false>(c, s, y, n, 0, st);
}

}  // namespace

hipError_t launch_dequant(int fmt, bool out_bf16, const uint8_t* codes, const uint8_t* scales,
                          void* y, int64_t n, int64_t cols, hipStream_t s) {
  switch (fmt) {
    case kE4M3: return by_out<kE4M3>(out_bf16, codes, scales, y, n, cols, s);
    case kE5M2: return by_out<kE5M2>(out_bf16, codes, scales, y, n, cols, s);
    case kE2M1: return by_out<kE2M1>(out_bf16, codes, scales, y, n, cols, s);
    case kE2M3: return by_out<kE2M3>(out_bf16, codes, scales, y, n, cols, s);
    case kE3M2: return by_out<kE3M2>(out_bf16, codes, scales, y, n, cols, s);
    case kInt8: return by_out<kInt8>(out_bf16, codes, scales, y, n, cols, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mx
