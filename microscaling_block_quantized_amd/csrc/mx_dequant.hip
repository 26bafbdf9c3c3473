// MX dequantization: codes + E8M0 scales -> FP32 or BF16.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §7: an E8M0 scale is a power of two, so
// applying it is an exponent add with no rounding; §2: scale code 0xFF is NaN
// and turns all 32 elements of its block NaN. Each value is formed exactly as
// an FP32 (every element value times 2^(k-127) is an FP32 number, subnormals
// included) by the gfx950 scaled up-conversion, and BF16 output is that FP32
// rounded to nearest-even. NaN is written as the positive quiet NaN.
//
// One thread handles 16 consecutive elements (half a block): a 16-byte (FP8)
// or 8-byte (E2M1) code load, one scale byte, and 64 or 32 bytes of output.
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kThreads = 256;

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

template <int F>
__device__ __forceinline__ void decode16(const uint32_t* cw, float sc, float* o) {
  if constexpr (F == kE2M1) {
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
      float2v lo, hi;
      if constexpr (F == kE4M3) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[d], sc, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[d], sc, true);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(cw[d], sc, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(cw[d], sc, true);
      }
      o[4 * d + 0] = lo.x; o[4 * d + 1] = lo.y; o[4 * d + 2] = hi.x; o[4 * d + 3] = hi.y;
    }
  }
}

template <int F, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             void* __restrict__ y, int64_t nchunks) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;   // 16-element chunk
  if (i >= nchunks) return;
  const uint32_t k = scales[i >> 1];
  uint32_t cw[4];
  if constexpr (F == kE2M1) {
    const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + i * 8));
    cw[0] = c.x; cw[1] = c.y; cw[2] = 0; cw[3] = 0;
  } else {
    const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + i * 16));
    cw[0] = c.x; cw[1] = c.y; cw[2] = c.z; cw[3] = c.w;
  }
  float o[16];
  decode16<F>(cw, scale_operand(k), o);
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

template <int F, bool B>
hipError_t launch_dq(const uint8_t* c, const uint8_t* s, void* y, int64_t n, hipStream_t st) {
  const int64_t chunks = n / 16;
  const int64_t blocks = (chunks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((mx_dequant_kernel<F, B>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, c, s, y,
                     chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(int fmt, bool out_bf16, const uint8_t* codes, const uint8_t* scales,
                          void* y, int64_t n, hipStream_t s) {
  switch (fmt) {
    case kE4M3: return out_bf16 ? launch_dq<kE4M3, true>(codes, scales, y, n, s)
                                : launch_dq<kE4M3, false>(codes, scales, y, n, s);
    case kE5M2: return out_bf16 ? launch_dq<kE5M2, true>(codes, scales, y, n, s)
                                : launch_dq<kE5M2, false>(codes, scales, y, n, s);
    default: return out_bf16 ? launch_dq<kE2M1, true>(codes, scales, y, n, s)
                             : launch_dq<kE2M1, false>(codes, scales, y, n, s);
  }
}

}  // namespace mx
