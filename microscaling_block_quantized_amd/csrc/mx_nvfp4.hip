// NVFP4 cast and dequantization.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §3, the §4 table and §7: E2M1 elements
// (the same as MXFP4's) in blocks of 16, each block with an unsigned E4M3
// (UE4M3, largest value 448) scale, and one FP32 global scale per tensor equal
// to the tensor's largest magnitude over 6 * 448. The codes are the exact ones:
//   g   = fp32(A / 2688)                (A: largest finite |x| of the batch slice)
//   s_b = UE4M3 nearest to amax_b / (6 g)   (exact quotient, RNE, saturating at 448)
//   q   = E2M1 nearest to x / (s_b g)       (exact quotient, RNE, saturating at 6)
//   y   = fp32(fp32(e2m1 * s_b) * g)    (dequantization; the first product is exact)
// A block whose scale code is 0, and every block when g is not a finite
// positive number, stores codes 0; a block holding NaN or Inf stores the UE4M3
// NaN code 0x7F and codes 0. Codes are packed as MXFP4's (element 2k in the low
// nibble); block scales are [B][R][C/16] and, for the column copy (the same
// cast of X^T), [B][C][R/16].
//
// g takes two launches and the cast: zero the caller's [B] FP32 array, then
// fold every workgroup's amax into it with one atomic max, as FP32 bits with
// the sign bit set (magnitudes order as unsigned integers, and the set sign
// marks a raw maximum). Each cast workgroup divides a marked value by 2688
// itself and writes g back, so any read sees either the mark or the same g.
// The cast reuses the MX tiled kernel's layout (128 x 256 tiles, 8 waves,
// LDS-staged column codes).
//
// The cast never divides per element and rarely per block, and decides every
// code exactly:
//  * Block code: estimated as fp32(amax_b * k), k = fp32(fp32(1/6) * fp32(1/g)),
//    within 4 FP32 ulps of the exact amax_b / (6 g) while amax_b >= 2^-120 and
//    2^-125 <= g <= 2^100. E4M3 rounding is monotone: when t - 16 ulps and
//    t + 16 ulps round to the same code, that is the code of the exact quotient
//    (t is first capped at 448: every quotient above it saturates to 448, and
//    the window then stays below E4M3's overflow). Any other block compares
//    amax_b with (midpoint x 6 g) in FP64, which is exact (at most 5 + 2 + 24
//    significant bits).
//  * Elements: r_b = fp32(1 / fp32(s_b g)) depends only on the block code, so
//    each workgroup divides once per code (256 entries in LDS). q' = fp32(x r_b)
//    is within 3 FP32 ulps of the exact quotient Q = x / (s_b g), which is not
//    enough near an E2M1 midpoint, and with BF16 inputs Q lands next to short
//    binary values often (g = fp32(A / 2688) has a periodic significand). So
//    every element is decided exactly, without a branch, on magnitudes: m = the
//    E4M3 value nearest to min(|q'|, 8) (the product clamped to [0, 1] with r_b
//    / 8, then one paired conversion dividing by 2^-3, and one back).
//    All E2M1 values and midpoints are E4M3 values, so when m is not a midpoint
//    |q'| and m round alike. sigma = fma(-(m s_b), g, |x|) has the exact sign
//    of |Q| - m (m s_b has at most 8 significant bits, and for
//    2^-90 <= g <= 2^100 a nonzero |x| - m s_b g is at least 2^-149 in
//    magnitude, so the one rounding keeps it nonzero). m moved by one FP32 ulp
//    towards |Q| (not at all when sigma is 0, an exact tie), with the sign of x,
//    then takes the hardware E2M1 rounding, which is the exact code: one ulp
//    above or below a midpoint rounds away from it, and an m that is not a
//    midpoint is a whole E4M3 step from every rounding boundary. With g outside that range every element compares
//    |x| with (midpoint x s_b g) in FP64 instead (exact: 3 + 4 + 24 bits).
#include "mx_cast_impl.h"

namespace mx {

namespace {

constexpr float kNvGlobalDiv = 6.0f * 448.0f;      // 2688
constexpr float kRcp6 = 0x1.555556p-3f;            // fp32(1/6)
constexpr uint32_t kNvWindow = 16;                 // ulps each side of the estimate
constexpr uint32_t kNvTcap = 0x43E00000u;          // 448: every t above it saturates alike, and
                                                   // 448 + 16 ulps stays below E4M3's overflow at 464
constexpr uint32_t kNvAmin = 0x03800000u;          // 2^-120: amax/6 stays a normal FP32
// global scales for which the element decision above is exact
constexpr float kNvGmin = 0x1p-90f, kNvGmax = 0x1p100f;

// ---------------- global scale ----------------

__global__ void nv_zero_kernel(uint32_t* gs, int64_t batch) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < batch) gs[i] = 0u;
}

constexpr int kAmaxThreads = 1024;
constexpr int kAmaxUnroll = 4;
// Workgroups over all slices: one per CU. The atomics of a persistent grid all
// arrive at the end, about 6 ns apart on one address, so fewer and larger
// workgroups win (measured at 16384 x 4096: 512 x 512 threads 72.2 us for the
// whole call, 256 x 1024 69.8 us, 1024 x 256 75.1 us).
constexpr int kAmaxBlocks = 256;
constexpr uint32_t kNvMark = 0x80000000u;

// Largest finite magnitude among a 16-byte chunk's elements, folded into m (FP32 bits).
template <bool BF16>
__device__ __forceinline__ uint32_t nv_fold(uint32_t m, const uint4& v) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = (&v.x)[d];
    if constexpr (BF16) {
      const uint32_t lo = (w & 0x7FFFu) << 16, hi = w & 0x7FFF0000u;
      m = max(m, lo < 0x7F800000u ? lo : 0u);
      m = max(m, hi < 0x7F800000u ? hi : 0u);
    } else {
      const uint32_t a = w & 0x7FFFFFFFu;
      m = max(m, a < 0x7F800000u ? a : 0u);
    }
  }
  return m;
}

// Largest finite |x| of batch slice blockIdx.y, marked, into amax[slice]: one
// atomic per workgroup. The loads are ordinary (cache-allocating) ones: the
// cast that follows reads the same bytes, and part of them are then still in
// the memory-side cache (measured: 9 us of 81 us at 16384 x 4096 BF16).
template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void nv_amax_kernel(const uint8_t* __restrict__ x, uint32_t* amax,
                                                                int64_t chunks_per_slice) {
  __shared__ uint32_t part[kAmaxThreads / 64];
  const uint8_t* xs = x + int64_t(blockIdx.y) * chunks_per_slice * 16;
  const int64_t stride = int64_t(gridDim.x) * kAmaxThreads;
  int64_t c = int64_t(blockIdx.x) * kAmaxThreads + threadIdx.x;
  uint32_t m = 0;
  for (; c + (kAmaxUnroll - 1) * stride < chunks_per_slice; c += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = *reinterpret_cast<const uint4*>(xs + (c + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = nv_fold<BF16>(m, v[u]);
  }
  for (; c < chunks_per_slice; c += stride) m = nv_fold<BF16>(m, *reinterpret_cast<const uint4*>(xs + c * 16));
  m = group_max<8>(m);
  m = max(m, dpp<kDppRor8>(m));
  m = max_xor32(max_xor16(m));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / 64; ++w) r = max(r, part[w]);
    atomicMax(amax + blockIdx.y, r | kNvMark);
  }
}

// ---------------- block scale and element encoding ----------------

struct NvBlock {
  uint32_t code;     // UE4M3 byte
  float rcp8;        // 1 / (8 s_b g): r_b / 8, exact (a power-of-two step)
  bool zero;         // store codes 0
};

// Per-slice constants of the block-code estimate.
struct NvScale {
  float g;           // global (decode) scale
  float k;           // fp32(fp32(1/6) * fp32(1/g))
  bool fast;         // 2^-125 <= g <= 2^100: the estimate's error bound holds
};

__device__ __forceinline__ NvScale nv_scale(float g) {
  NvScale s;
  s.g = g;
  s.fast = g >= 0x1p-125f && g <= 0x1p100f;
  s.k = kRcp6 * (1.0f / (s.fast ? g : 1.0f));
  return s;
}

// The block a partner lane computed: code and reciprocal arrive through a lane
// exchange, the zero flag is recomputed.
__device__ __forceinline__ NvBlock nv_block_of(uint32_t code, uint32_t rcp_bits) {
  NvBlock b;
  b.code = code;
  b.rcp8 = __uint_as_float(rcp_bits);
  b.zero = b.rcp8 != b.rcp8;
  return b;
}

// c ? x : y, field by field (one select each; a select of whole structs can
// end up in private memory)
__device__ __forceinline__ NvBlock nv_pick(bool c, const NvBlock& x, const NvBlock& y) {
  NvBlock r;
  r.code = c ? x.code : y.code;
  r.rcp8 = c ? x.rcp8 : y.rcp8;
  r.zero = c ? x.zero : y.zero;
  return r;
}

// UE4M3 value of code c (0 .. 0x7E) in FP64: subnormals m * 2^-9, normals (8 + m) * 2^(e - 10).
__device__ __forceinline__ double ue4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return __builtin_ldexp(double(e == 0 ? m : 8u + m), e == 0 ? -9 : int(e) - 10);
}

// The defining computation: the UE4M3 code nearest to amax / (6 g), ties to the
// even code, saturating at 0x7E (448). Midpoint i lies between codes i and
// i + 1, and the code is the number of midpoints the quotient passes (strictly
// above, or on one whose upper neighbour is even), found by binary search over
// exact FP64 comparisons of amax with (midpoint x 6 g) (at most 5 + 2 + 24
// significant bits). amag: FP32 bits of the block's largest magnitude
// (>= 0x7F800000: NaN or Inf present).
__device__ __forceinline__ uint32_t nv_code_exact(uint32_t amag, float g) {
  if (amag >= 0x7F800000u) return 0x7Fu;
  if (!(g > 0.0f && g < __builtin_inff())) return 0u;
  const double num = double(__uint_as_float(amag));
  const double den = 6.0 * double(g);                  // exact: 2 + 24 bits
  uint32_t lo = 0, hi = 0x7Eu;
#pragma unroll 1
  while (lo < hi) {
    const uint32_t i = (lo + hi) >> 1;
    const double t = 0.5 * (ue4m3_value(i) + ue4m3_value(i + 1)) * den;
    const bool up = num > t || (num == t && (i & 1u));
    lo = up ? i + 1 : lo;
    hi = up ? hi : i;
  }
  return lo;
}

// The same code through the estimate, falling back to nv_code_exact.
// A zero block (amag 0) estimates t = 0 and codes 0 through the same window;
// NaN / Inf blocks (amag >= 0x7F800000) take 0x7F.
__device__ __forceinline__ uint32_t nv_code(uint32_t amag, const NvScale& s) {
  const uint32_t tb = min(__float_as_uint(__uint_as_float(amag) * s.k), kNvTcap);
  const uint32_t lo = tb > kNvWindow ? tb - kNvWindow : 0u;
  const uint32_t w = cvt2_f32<kE4M3, false>(tb, __uint_as_float(lo), __uint_as_float(tb + kNvWindow),
                                            scale_operand(127u));
  const uint32_t c0 = w & 0xFFu, c1 = (w >> 8) & 0xFFu;
  const bool special = amag >= 0x7F800000u;
  // fast: amag == 0 or amag >= 2^-120 (one unsigned compare), and both ends agree
  const bool slow = !special && !(s.fast && amag - 1u >= kNvAmin - 1u && c0 == c1);
  uint32_t c = special ? 0x7Fu : c0;
  if (slow) c = nv_code_exact(amag, s.g);
  return c;
}

// LDS table of fp32(1 / fp32(s_c * g)) / 8 for every scale byte c (g in
// [2^-90, 2^100], so the quotient stays normal and the division by 8 is exact);
// NaN marks the codes whose blocks store codes 0 (c == 0 and the NaN code 0x7F).
constexpr int kNvTab = 256;
__device__ __forceinline__ void nv_fill_table(float* tab, float g) {
  const int c = threadIdx.x;
  if (c < kNvTab) {
    const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uint32_t(c), scale_operand(127u), false)[0];
    const float r = (1.0f / (s * g)) * 0.125f;
    tab[c] = (c == 0 || c == 0x7F) ? __builtin_nanf("") : r;
  }
}

__device__ __forceinline__ NvBlock nv_block(uint32_t amag, const NvScale& s, const float* tab) {
  NvBlock b;
  b.code = nv_code(amag, s);
  b.rcp8 = tab[b.code];
  b.zero = b.rcp8 != b.rcp8;
  return b;
}

// E2M1 code of x / (s_b g), decided exactly: binary search for the number of
// midpoints |x| passes, comparing with (midpoint x s_b g) in FP64 (exact: at
// most 3 + 4 + 24 bits); on a midpoint, up when the upper neighbour's code is
// even (midpoints 1, 3 and 5). The midpoints are 2^-2 * (1, 3, 5, 7, 10, 14, 20),
// packed as 5-bit fields of kNvMid4.
constexpr uint64_t kNvMid4 = 1ull | 3ull << 5 | 5ull << 10 | 7ull << 15 | 10ull << 20 | 14ull << 25 | 20ull << 30;
__device__ __forceinline__ uint32_t nv_code1_exact(float f, double d) {
  const double a = __builtin_fabs(double(f));
  uint32_t lo = 0, hi = 7;
#pragma unroll 1
  while (lo < hi) {
    const uint32_t i = (lo + hi) >> 1;
    const double t = double(uint32_t(kNvMid4 >> (5 * i)) & 31u) * 0.25 * d;
    const bool up = a > t || (a == t && (i & 1u));
    lo = up ? i + 1 : lo;
    hi = up ? hi : i;
  }
  return lo | ((__float_as_uint(f) >> 28) & 8u);
}

// One element's exactly rounded quotient stand-in (see the header), worked on
// magnitudes: m, the E4M3 value nearest to min(|q'|, 8), moved by one FP32 ulp
// towards |x| / (s_b g) (not at all at an exact tie), then given the sign of x
// (so that -0 and tiny negative x code as -0; the E2M1 conversion keeps the
// sign of zero and subnormal inputs). sigma is never -0: the sum of |x| and a
// product of sign <= 0 that is exactly zero rounds to +0, so its bits read as
// an integer are positive for sigma > 0, 0 for a tie and negative for sigma < 0.
// m = 0 only moves up (to the smallest subnormal, which codes as 0).
__device__ __forceinline__ float nv_nudged(float f, float m, float ms, float g) {
  const float sigma = __builtin_fmaf(-ms, g, __builtin_fabsf(f));   // exact sign of |x| - m s_b g
  // clamp of sigma's bits to [-1, 1] as one v_med3_i32 (written out: the compiler
  // turns the min / max form into two compares and two selects)
  int step;
  asm("v_med3_i32 %0, %1, -1, 1" : "=v"(step) : "v"(sigma));
  return __builtin_copysignf(__uint_as_float(__float_as_uint(m) + uint32_t(step)), f);
}

// Four FP32 values -> four E2M1 codes in the low 16 bits, each the exact
// rounding of x / (s_b g) (see the header).
__device__ __forceinline__ uint32_t nv_encode4(float f0, float f1, float f2, float f3, const NvBlock& b,
                                               float g) {
  const float one = scale_operand(127u);
  const float eighth = scale_operand(124u);                     // the conversion divides by 2^-3
  const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b.code, one, false)[0];
  // min(|x| r_b, 8) / 8 as the product's clamp to [0, 1] (a NaN r_b, a zero
  // block, gives 0; its codes are dropped below)
  const float q0 = __builtin_amdgcn_fmed3f(__builtin_fabsf(f0) * b.rcp8, 0.0f, 1.0f);
  const float q1 = __builtin_amdgcn_fmed3f(__builtin_fabsf(f1) * b.rcp8, 0.0f, 1.0f);
  const float q2 = __builtin_amdgcn_fmed3f(__builtin_fabsf(f2) * b.rcp8, 0.0f, 1.0f);
  const float q3 = __builtin_amdgcn_fmed3f(__builtin_fabsf(f3) * b.rcp8, 0.0f, 1.0f);
  // nearest E4M3 values of 8 q (no overflow at 8); the two conversions fill all
  // four bytes, so the register they start from is immaterial
  uint32_t e = cvt2_f32<kE4M3, false>(__float_as_uint(q0), q0, q1, eighth);
  e = cvt2_f32<kE4M3, true>(e, q2, q3, eighth);
  const float2v m01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, one, false);
  const float2v m23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, one, true);
  uint32_t w = cvt2_fp4_f32<0>(e, nv_nudged(f0, m01.x, m01.x * s, g), nv_nudged(f1, m01.y, m01.y * s, g), one);
  w = cvt2_fp4_f32<1>(w, nv_nudged(f2, m23.x, m23.x * s, g), nv_nudged(f3, m23.y, m23.y * s, g), one);
  return b.zero ? 0u : (w & 0xFFFFu);
}

// Eight FP32 values of one block -> eight E2M1 codes filling a dword (element
// i in bits 4i+3 .. 4i), each decided as in nv_encode4.
__device__ __forceinline__ uint32_t nv_encode8(float f0, float f1, float f2, float f3, float f4, float f5, float f6,
                                               float f7, const NvBlock& b, float g) {
  const float one = scale_operand(127u);
  const float eighth = scale_operand(124u);
  const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b.code, one, false)[0];
  auto q = [&](float f) { return __builtin_amdgcn_fmed3f(__builtin_fabsf(f) * b.rcp8, 0.0f, 1.0f); };
  const float q0 = q(f0), q1 = q(f1), q2 = q(f2), q3 = q(f3), q4 = q(f4), q5 = q(f5), q6 = q(f6), q7 = q(f7);
  uint32_t e0 = cvt2_f32<kE4M3, false>(__float_as_uint(q0), q0, q1, eighth);
  e0 = cvt2_f32<kE4M3, true>(e0, q2, q3, eighth);
  uint32_t e1 = cvt2_f32<kE4M3, false>(__float_as_uint(q4), q4, q5, eighth);
  e1 = cvt2_f32<kE4M3, true>(e1, q6, q7, eighth);
  const float2v m01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e0, one, false);
  const float2v m23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e0, one, true);
  const float2v m45 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e1, one, false);
  const float2v m67 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e1, one, true);
  uint32_t w = cvt2_fp4_f32<0>(e0, nv_nudged(f0, m01.x, m01.x * s, g), nv_nudged(f1, m01.y, m01.y * s, g), one);
  w = cvt2_fp4_f32<1>(w, nv_nudged(f2, m23.x, m23.x * s, g), nv_nudged(f3, m23.y, m23.y * s, g), one);
  w = cvt2_fp4_f32<2>(w, nv_nudged(f4, m45.x, m45.x * s, g), nv_nudged(f5, m45.y, m45.y * s, g), one);
  w = cvt2_fp4_f32<3>(w, nv_nudged(f6, m67.x, m67.x * s, g), nv_nudged(f7, m67.y, m67.y * s, g), one);
  return b.zero ? 0u : w;
}

// One 16-element block decided entirely in FP64 (g outside [2^-90, 2^100], or
// not a finite positive number): 16 elements at stride `step` elements from p,
// the 8 code bytes to `codes` (8-byte aligned) and the scale byte to `scale`.
template <bool BF16>
__device__ __forceinline__ void nv_block_exact(const uint8_t* p, int64_t step, float g, uint8_t* codes,
                                               uint8_t* scale) {
  float f[16];
  uint32_t amag = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (BF16) {
      f[i] = __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t*>(p + i * step * 2)) << 16);
    } else {
      f[i] = *reinterpret_cast<const float*>(p + i * step * 4);
    }
    amag = max(amag, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  }
  const uint32_t code = nv_code_exact(amag, g);
  const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code, scale_operand(127u), false)[0];
  const double d = double(s) * double(g);                       // exact: 4 + 24 bits
  const bool zero = code == 0 || code == 0x7F;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= (zero ? 0u : nv_code1_exact(f[i], d)) << (4 * (i & 7));
  *reinterpret_cast<uint2*>(codes) = make_uint2(w[0], w[1]);
  *scale = uint8_t(code);
}

// ---------------- cast ----------------

template <bool BF16, int AX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 2))) void nv_cast_kernel(NvArgs a) {
  constexpr int VEC = InC<BF16>::vec;          // elements per 16-byte chunk: 8 | 4
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int LPR = 128 / VEC;               // lanes per 128-column wave row: 16 | 32
  constexpr int RG = 64 / LPR;                 // row groups per wave: 4 | 2
  constexpr int RPT = 32 / RG;                 // rows per thread: 8 | 16
  constexpr int LPB = 16 / VEC;                // lanes per 16-element row block: 2 | 4
  constexpr int HALF = 4 * LPB;                // lanes covering 4 row blocks (one scale dword): 8 | 16
  constexpr bool ROWS = (AX & kRow) != 0;
  constexpr bool COLS = (AX & kCol) != 0;
  constexpr int BPC = kTileR / 2;              // staged code bytes per tile column (4-bit codes): 64
  constexpr int CPC = BPC / 16;                // 16-byte chunks per staged column: 4
  constexpr int SPC = kTileR / 16;             // column blocks (scales) per tile column: 8

  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[COLS ? kTileC * BPC : 16];
  // column-block scale codes as [16-row group][tile column]: a lane's codes of its VEC
  // columns are contiguous and leave in one store
  __shared__ __attribute__((aligned(8))) uint8_t lds_scales[COLS ? kTileC * SPC : 8];
  __shared__ float lds_rtab[kNvTab];
  // With both copies, a wave row's row codes (64 bytes, half of a 128-byte line) are
  // staged as [tile row][128 bytes] and written as whole lines after the barrier the
  // column copy needs anyway; chunk index XORed with (row / 8) mod 8 against bank
  // conflicts between the row groups of a wave.
  constexpr bool ROWLDS = ROWS && COLS;
  __shared__ __attribute__((aligned(16))) uint8_t lds_rows[ROWLDS ? kTileR * kTileC / 2 : 16];
  // Row scales of full-width tiles (kNvRowScaleWords): a tile row's 16 scale
  // bytes (4 dwords from 2 waves) are staged and leave as one 16-byte store
  // after the barrier.
  // one row's 4 scale dwords at a 5-dword pitch: the 8 lanes storing rows 8 apart then reach
  // different banks
  __shared__ __attribute__((aligned(16))) uint32_t lds_rs[ROWLDS ? kTileR * 5 : 4];
  auto rows_off = [](int r, int c) { return r * (kTileC / 2) + ((c / 2) ^ (((r >> 3) & 7) << 4)); };

  uint32_t bi, tr, tcol;
  tile_coords(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_c, false, bi, tr, tcol);
  const int64_t R = a.rows, C = a.cols;
  const int64_t r0 = int64_t(tr) * kTileR;
  const int64_t c0 = int64_t(tcol) * kTileC;
  const int rows_in = int(min<int64_t>(R - r0, kTileR));
  const int cols_in = int(min<int64_t>(C - c0, kTileC));
  const uint32_t Cu = uint32_t(C);
  const bool rs16 = ROWLDS && (a.flags & kNvRowScaleWords) != 0;
  // a marked value is the slice's raw amax: divide it here and publish g
  const uint32_t gbits = __float_as_uint(a.global_scale[bi]);
  float g = __uint_as_float(gbits);
  if ((a.flags & kNvMarkedAmax) && (gbits & kNvMark)) {
    g = __uint_as_float(gbits & ~kNvMark) / kNvGlobalDiv;
    if (threadIdx.x == 0) a.global_scale[bi] = g;
  }

  const int64_t tile_elem = (int64_t(bi) * R + r0) * C + c0;
  const uint8_t* xt = reinterpret_cast<const uint8_t*>(a.x) + tile_elem * ES;
  if (!(g >= kNvGmin && g <= kNvGmax)) {
    // g outside [2^-90, 2^100] (or 0, negative, Inf, NaN): the whole slice is
    // decided in FP64, one 16-element block per thread at a time
    const int rb_row = cols_in / 16, rb_col = rows_in / 16;
    if constexpr (ROWS) {
#pragma unroll 1
      for (int i = threadIdx.x; i < rows_in * rb_row; i += kThreads) {
        const int r = i / rb_row, cb = i - r * rb_row;
        const int64_t e = (int64_t(bi) * R + r0 + r) * C + c0 + 16 * cb;
        nv_block_exact<BF16>(xt + (int64_t(r) * C + 16 * cb) * ES, 1, g,
                             reinterpret_cast<uint8_t*>(a.row_codes) + e / 2, a.row_scales + e / 16);
      }
    }
    if constexpr (COLS) {
#pragma unroll 1
      for (int i = threadIdx.x; i < cols_in * rb_col; i += kThreads) {
        const int c = i / rb_col, rb = i - c * rb_col;
        const int64_t e = (int64_t(bi) * C + c0 + c) * R + r0 + 16 * rb;
        nv_block_exact<BF16>(xt + (int64_t(16 * rb) * C + c) * ES, C, g,
                             reinterpret_cast<uint8_t*>(a.col_codes) + e / 2, a.col_scales + e / 16);
      }
    }
    return;
  }

  const int wid = threadIdx.x >> 6;
  const int wr = wid % kWaveRows, wc = wid / kWaveRows;
  const int lane = threadIdx.x & 63;
  const int q = lane / LPR, t = lane % LPR;
  const int lcol = 128 * wc + t * VEC;
  const int lrow = 32 * wr + RPT * q;
  const bool col_ok = lcol < cols_in;

  const uint32_t xoff = (uint32_t(lrow) * Cu + uint32_t(lcol)) * ES;
  uint4 v[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const bool ok = col_ok && lrow + k < rows_in;
    const uint4 d = load_nt(xt + (ok ? xoff + uint32_t(k) * Cu * ES : 0u));
    v[k] = ok ? d : make_uint4(0u, 0u, 0u, 0u);
  }
  const NvScale sc = nv_scale(g);
  nv_fill_table(lds_rtab, g);
  __syncthreads();

  // element e (0 .. VEC-1) of row k as FP32
  auto elem = [&](int k, int e) -> float {
    if constexpr (BF16) {
      const uint32_t w = (&v[k].x)[e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
      return __uint_as_float((&v[k].x)[e]);
    }
  };

  // column blocks: 16 rows = this thread's rows (FP32) or those of two row groups (BF16)
  NvBlock cb[COLS ? VEC : 1];
  if constexpr (COLS) {
    if constexpr (BF16) {
      uint32_t cm[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = (&v[0].x)[d] & 0x7FFF7FFFu;
#pragma unroll
      for (int k = 1; k < RPT; ++k) {
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], (&v[k].x)[d] & 0x7FFF7FFFu);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = pk_max_xor16(cm[d]);   // row groups q and q ^ 1
      // Row groups q and q ^ 1 share their 8 column blocks: the even one codes
      // blocks 0..3, the odd one 4..7, and they swap the results. v_permlane16_swap
      // of (x, x) gives, in an even 16-lane row, (own, partner) and in an odd
      // one (partner, own).
      const bool qodd = (q & 1) != 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        auto amag = [&](int jj) { return (jj & 1) ? (cm[jj >> 1] & 0xFFFF0000u) : (cm[jj >> 1] << 16); };
        const uint32_t a_lo = amag(j), a_hi = amag(j + 4);
        const NvBlock mine = nv_block(qodd ? a_hi : a_lo, sc, lds_rtab);
        const auto xc = __builtin_amdgcn_permlane16_swap(mine.code, mine.code, false, false);
        const uint32_t rb = __float_as_uint(mine.rcp8);
        const auto xr = __builtin_amdgcn_permlane16_swap(rb, rb, false, false);
        const NvBlock other = nv_block_of(qodd ? uint32_t(xc[0]) : uint32_t(xc[1]),
                                          qodd ? uint32_t(xr[0]) : uint32_t(xr[1]));
        cb[j] = nv_pick(qodd, other, mine);
        cb[j + 4] = nv_pick(qodd, mine, other);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t m = (&v[0].x)[d] & 0x7FFFFFFFu;
#pragma unroll
        for (int k = 1; k < RPT; ++k) m = max(m, (&v[k].x)[d] & 0x7FFFFFFFu);
        cb[d] = nv_block(m, sc, lds_rtab);
      }
    }
  }

  // ---------------- row-wise blocks ----------------
  if constexpr (ROWS) {
    uint8_t* rct = reinterpret_cast<uint8_t*>(a.row_codes) + tile_elem / 2;
    const uint32_t rcoff = (uint32_t(lrow) * Cu + uint32_t(lcol)) / 2;
    // the scale dword of blocks 4d .. 4d+3 of the wave's 128 columns, stored by lane t = HALF * d
    const int dcol = 128 * wc + 64 * (t / HALF);
    uint8_t* sdst = a.row_scales + ((int64_t(bi) * R + r0 + lrow) * C + c0 + dcol) / 16;
    // BF16: lanes t and t ^ 1 hold the two halves of each row block; of a pair of
    // rows the even lane codes the first block and the odd lane the second, and
    // they swap the results (the second waits in `pend` for the next row)
    auto bf16_row_max = [&](int k) {
      const uint32_t h = pk_max_u16(pk_max_u16(v[k].x & 0x7FFF7FFFu, v[k].y & 0x7FFF7FFFu),
                                    pk_max_u16(v[k].z & 0x7FFF7FFFu, v[k].w & 0x7FFF7FFFu));
      const uint32_t m = max(h & 0xFFFFu, h >> 16) << 16;
      return max(m, dpp<kDppXor1>(m));
    };
    NvBlock pend;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      NvBlock blk;
      if constexpr (BF16) {
        if ((k & 1) == 0) {
          // both maxima on every lane first: each takes a lane exchange, which the
          // partner lane must execute too
          const bool todd = (t & 1) != 0;
          const uint32_t m0 = bf16_row_max(k), m1 = bf16_row_max(k + 1);
          const NvBlock mine = nv_block(todd ? m1 : m0, sc, lds_rtab);
          const NvBlock other = nv_block_of(dpp<kDppXor1>(mine.code), dpp<kDppXor1>(__float_as_uint(mine.rcp8)));
          blk = nv_pick(todd, other, mine);
          pend = nv_pick(todd, mine, other);
        } else {
          blk = pend;
        }
      } else {
        uint32_t m = max(max(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu), max(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu));
        m = group_max<4>(m);
        blk = nv_block(m, sc, lds_rtab);
      }
      const bool ok = col_ok && lrow + k < rows_in;
      uint8_t* dst = rct + rcoff + uint32_t(k) * Cu / 2;
      if constexpr (BF16) {
        const uint32_t w = nv_encode8(elem(k, 0), elem(k, 1), elem(k, 2), elem(k, 3), elem(k, 4), elem(k, 5),
                                      elem(k, 6), elem(k, 7), blk, g);
        if constexpr (ROWLDS) *reinterpret_cast<uint32_t*>(lds_rows + rows_off(lrow + k, lcol)) = w;
        else if (ok) store_nt4(dst, w);
      } else {
        const uint32_t w = nv_encode4(elem(k, 0), elem(k, 1), elem(k, 2), elem(k, 3), blk, g);
        if constexpr (ROWLDS) *reinterpret_cast<uint16_t*>(lds_rows + rows_off(lrow + k, lcol)) = uint16_t(w);
        else if (ok) store_nt2(dst, w);
      }
      // OR the codes of the 4 blocks of each group of HALF lanes into one dword that every
      // lane of the group holds: BF16 pairs lanes 2 apart (quad_perm), then the two halves
      // of each 8-lane group (row_half_mirror); FP32 rotates its 16-lane row by 4 and 8
      uint32_t sb = blk.code << (8 * ((t / LPB) & 3));
      if constexpr (BF16) {
        sb |= dpp<kDppXor2>(sb);
        sb |= dpp<kDppHalfMirror>(sb);
      } else {
        sb |= dpp<kDppRor4>(sb);
        sb |= dpp<kDppRor8>(sb);
      }
      if (rs16) {
        if (t % HALF == 0) lds_rs[(lrow + k) * 5 + dcol / 64] = sb;
      } else if (t % HALF == 0 && lrow + k < rows_in && dcol < cols_in) {
        uint8_t* dst = sdst + int64_t(k) * C / 16;
        if (a.flags & kRowScaleDword) {
          *reinterpret_cast<uint32_t*>(dst) = sb;
        } else {
#pragma unroll
          for (int m2 = 0; m2 < 4; ++m2)
            if (dcol + 16 * m2 < cols_in) dst[m2] = uint8_t(sb >> (8 * m2));
        }
      }
    }
  }

  // ---------------- column-wise blocks ----------------
  if constexpr (COLS) {
    const int byte0 = lrow / 2;                       // this thread's offset inside a staged column
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const int cl = lcol + j;
      // BF16: 4-byte writes; the 4-byte slot inside a chunk is XORed with (column / 32) mod 4 so
      // that a quarter-wave's 16 columns reach 16 different banks
      const int slot = BF16 ? ((cl >> 5) & 3) << 2 : 0;
      const int off = cl * BPC + ((((byte0 >> 4) ^ ((cl >> 3) & (CPC - 1))) << 4) | ((byte0 & 15) ^ slot));
      if constexpr (BF16) {
        const uint32_t w = nv_encode8(elem(0, j), elem(1, j), elem(2, j), elem(3, j), elem(4, j), elem(5, j),
                                      elem(6, j), elem(7, j), cb[j], g);
        *reinterpret_cast<uint32_t*>(lds_codes + off) = w;               // 8 rows in 4 bytes
      } else {
        uint32_t w[2];
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8)
          w[h8] = nv_encode8(elem(8 * h8, j), elem(8 * h8 + 1, j), elem(8 * h8 + 2, j), elem(8 * h8 + 3, j),
                             elem(8 * h8 + 4, j), elem(8 * h8 + 5, j), elem(8 * h8 + 6, j), elem(8 * h8 + 7, j), cb[j], g);
        *reinterpret_cast<uint2*>(lds_codes + off) = make_uint2(w[0], w[1]);
      }
    }
    // column block index inside the tile: 16-row groups
    if (BF16 ? (q % 2 == 0) : true) {
      if constexpr (VEC == 8) {
        *reinterpret_cast<uint2*>(lds_scales + (lrow / 16) * kTileC + lcol) =
            make_uint2(pack_low_bytes(cb[0].code, cb[1].code, cb[2].code, cb[3].code),
                       pack_low_bytes(cb[4].code, cb[5].code, cb[6].code, cb[7].code));
      } else {
        *reinterpret_cast<uint32_t*>(lds_scales + (lrow / 16) * kTileC + lcol) =
            pack_low_bytes(cb[0].code, cb[1].code, cb[2].code, cb[3].code);
      }
    }
    __syncthreads();

    const uint32_t Ru = uint32_t(R);
    const uint32_t cpitch = Ru / 2;                   // column-plane row pitch in bytes
    const int64_t ctile_elem = (int64_t(bi) * C + c0) * R + r0;
    uint8_t* cct = reinterpret_cast<uint8_t*>(a.col_codes) + ctile_elem / 2;
#pragma unroll
    for (int i = 0; i < kTileC * CPC / kThreads; ++i) {
      const int id = threadIdx.x + i * kThreads;
      const int cl = id / CPC;
      const int part = id % CPC;                      // rows 32 part .. +31
      if (cl < cols_in && 32 * part < rows_in) {
        uint4 w = *reinterpret_cast<const uint4*>(lds_codes + cl * BPC + ((part ^ ((cl >> 3) & (CPC - 1))) << 4));
        if constexpr (BF16) {
          // undo the slot XOR: column cl = (threadIdx.x + 512 i) / 4 has (cl / 32) mod 4 = (threadIdx.x / 128) mod 4
          const int p = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 7) & 3);
          if (p & 1) w = make_uint4(w.y, w.x, w.w, w.z);
          if (p & 2) w = make_uint4(w.z, w.w, w.x, w.y);
        }
        uint8_t* dst = cct + uint32_t(cl) * cpitch + uint32_t(part) * 16;
        if (32 * part + 32 > rows_in) {
          store_nt8(dst, make_uint2(w.x, w.y));        // a 16-row tail
        } else if (Ru % 32 == 0) {
          store_nt16(dst, w);
        } else {                                       // rows of R/2 bytes are only 8-byte aligned
          store_nt8(dst, make_uint2(w.x, w.y));
          store_nt8(dst + 8, make_uint2(w.z, w.w));
        }
      }
    }
    if constexpr (ROWLDS) {
      // the staged row codes: 8 lanes per tile row, 16 bytes (32 columns) each; a
      // ragged last chunk holds 16 columns, and rows of C/2 bytes with C % 32 != 0
      // are only 8-byte aligned
      uint8_t* rct = reinterpret_cast<uint8_t*>(a.row_codes) + tile_elem / 2;
#pragma unroll
      for (int i = 0; i < kTileR * 8 / kThreads; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int rl = id >> 3, part = id & 7;
        if (rl < rows_in && 32 * part < cols_in) {
          const uint4 w = *reinterpret_cast<const uint4*>(lds_rows + rl * (kTileC / 2) + ((part ^ ((rl >> 3) & 7)) << 4));
          uint8_t* dst = rct + uint32_t(rl) * (Cu / 2) + uint32_t(16 * part);
          if (32 * part + 32 > cols_in) {
            store_nt8(dst, make_uint2(w.x, w.y));
          } else if (Cu % 32 == 0) {
            store_nt16(dst, w);
          } else {
            store_nt8(dst, make_uint2(w.x, w.y));
            store_nt8(dst + 8, make_uint2(w.z, w.w));
          }
        }
      }
    }
    if (rs16 && int(threadIdx.x) < rows_in) {
      const int rl = threadIdx.x;
      uint8_t* dst = a.row_scales + ((int64_t(bi) * R + r0 + rl) * C + c0) / 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(lds_rs[rl * 5], lds_rs[rl * 5 + 1], lds_rs[rl * 5 + 2], lds_rs[rl * 5 + 3]);
    }
    if (int(threadIdx.x) < cols_in) {
      const int cl = threadIdx.x;
      uint8_t* dst = a.col_scales + ctile_elem / 16 + uint32_t(cl) * Ru / 16;
      if ((a.flags & kColScaleDword) && rows_in == kTileR) {
        auto codes4 = [&](int s0) {
          return uint32_t(lds_scales[s0 * kTileC + cl]) | (uint32_t(lds_scales[(s0 + 1) * kTileC + cl]) << 8) |
                 (uint32_t(lds_scales[(s0 + 2) * kTileC + cl]) << 16) | (uint32_t(lds_scales[(s0 + 3) * kTileC + cl]) << 24);
        };
        *reinterpret_cast<uint32_t*>(dst) = codes4(0);
        *reinterpret_cast<uint32_t*>(dst + 4) = codes4(4);
      } else {
#pragma unroll
        for (int s = 0; s < SPC; ++s)
          if (16 * s < rows_in) dst[s] = lds_scales[s * kTileC + cl];
      }
    }
  }
}

template <bool BF16, int AX>
hipError_t launch_nv_cast(const NvArgs& a, uint32_t nblocks, hipStream_t s) {
  return launch_kernel(nv_cast_kernel<BF16, AX>, dim3(nblocks), dim3(kThreads), s, a);
}

template <bool BF16>
hipError_t nv_by_axis(int axis, const NvArgs& a, uint32_t nb, hipStream_t s) {
  switch (axis) {
    case kRow: return launch_nv_cast<BF16, kRow>(a, nb, s);
    case kCol: return launch_nv_cast<BF16, kCol>(a, nb, s);
    default: return launch_nv_cast<BF16, kBoth>(a, nb, s);
  }
}

// ---------------- dequantization ----------------

constexpr int kDqThreads = 256;

// One thread per 16-element block: 8 code bytes, one scale byte, g of its slice.
template <bool OUT_BF16>
__global__ __launch_bounds__(kDqThreads) void nv_dequant_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                const float* __restrict__ gs, void* __restrict__ y,
                                                                int64_t nblocks, int64_t blocks_per_slice) {
  const int64_t i = int64_t(blockIdx.x) * kDqThreads + threadIdx.x;
  if (i >= nblocks) return;
  const uint32_t k = scales[i];
  const float g = gs[i / blocks_per_slice];
  const float one = scale_operand(127u);
  const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(k, one, false)[0];
  const uint2 c = *reinterpret_cast<const uint2*>(codes + i * 8);
  float o[16];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t cw = d ? c.y : c.x;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float2v e;
      switch (p) {
        case 0: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, one, 0); break;
        case 1: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, one, 1); break;
        case 2: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, one, 2); break;
        default: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, one, 3); break;
      }
      o[8 * d + 2 * p] = (e.x * s) * g;
      o[8 * d + 2 * p + 1] = (e.y * s) * g;
    }
  }
  const bool nan = (k & 0x7Fu) == 0x7Fu;
  uint32_t ob[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t b = __float_as_uint(o[e]);
    ob[e] = (nan || (b & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : b;
  }
  if constexpr (OUT_BF16) {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16x2 p = {static_cast<__bf16>(__uint_as_float(ob[2 * e])), static_cast<__bf16>(__uint_as_float(ob[2 * e + 1]))};
      uint32_t w = __builtin_bit_cast(uint32_t, p);
      w = ob[2 * e] == 0x7FC00000u ? ((w & 0xFFFF0000u) | 0x7FC0u) : w;
      w = ob[2 * e + 1] == 0x7FC00000u ? ((w & 0x0000FFFFu) | 0x7FC00000u) : w;
      h[e] = w;
    }
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(y) + i * 32);
    dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
    dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(y) + i * 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = make_uint4(ob[4 * e], ob[4 * e + 1], ob[4 * e + 2], ob[4 * e + 3]);
  }
}

}  // namespace

hipError_t launch_nvfp4_global(bool in_bf16, const void* x, int64_t batch, int64_t slice_elems, float* gs,
                               hipStream_t s) {
  uint32_t* gb = reinterpret_cast<uint32_t*>(gs);
  const uint32_t small = uint32_t((batch + 255) / 256);
  const hipError_t e = launch_kernel(nv_zero_kernel, dim3(small), dim3(256), s, gb, batch);
  if (e != hipSuccess) return e;
  const int64_t chunks = slice_elems * (in_bf16 ? 2 : 4) / 16;
  const int64_t per_block = int64_t(kAmaxThreads) * kAmaxUnroll;
  const int64_t want = (chunks + per_block - 1) / per_block;
  const int64_t cap = batch >= kAmaxBlocks ? 1 : kAmaxBlocks / batch;
  const dim3 grid(uint32_t(want < cap ? want : cap), uint32_t(batch));
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  return in_bf16 ? launch_kernel(nv_amax_kernel<true>, grid, dim3(kAmaxThreads), s, xb, gb, chunks)
                 : launch_kernel(nv_amax_kernel<false>, grid, dim3(kAmaxThreads), s, xb, gb, chunks);
}

hipError_t launch_nvfp4_cast(bool in_bf16, int axis, const NvArgs& a, uint32_t nblocks, hipStream_t s) {
  return in_bf16 ? nv_by_axis<true>(axis, a, nblocks, s) : nv_by_axis<false>(axis, a, nblocks, s);
}

hipError_t launch_nvfp4_dequant(bool out_bf16, const uint8_t* codes, const uint8_t* scales, const float* gs,
                                void* y, int64_t nblocks, int64_t blocks_per_slice, hipStream_t s) {
  const uint32_t grid = uint32_t((nblocks + kDqThreads - 1) / kDqThreads);
  return out_bf16 ? launch_kernel(nv_dequant_kernel<true>, dim3(grid), dim3(kDqThreads), s, codes, scales, gs, y,
                                  nblocks, blocks_per_slice)
                  : launch_kernel(nv_dequant_kernel<false>, dim3(grid), dim3(kDqThreads), s, codes, scales, gs, y,
                                  nblocks, blocks_per_slice);
}

}  // namespace mx
