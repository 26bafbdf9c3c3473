// FP4-in-FP8 nested requantization.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §6 (DeepSeek-V4's nested structure):
// MXFP4 weights (1x32 tiles with E8M0 scales) are dequantized into FP8 E4M3
// whose scales are per 128x128 tile, which holds 512 of the 1x32 tiles; the
// conversion is lossless while, inside each 128x128 tile, the largest and the
// smallest 1x32 scale stay within a bounded ratio, a property of the weights
// that has to be checked. The arithmetic fixed here:
//   * a 1x32 sub-block is active when one of its codes has a nonzero
//     magnitude and its scale is not 0xFF; kmax / kmin are the largest and
//     smallest scale codes of the block's active sub-blocks;
//   * the block scale is S = 2^(kmax - 133), so E2M1's 6 of the largest
//     sub-block lands on 384 (S = 1 for a block with no active sub-block);
//   * element v = e2m1 * 2^(k - 127) is stored as E4M3(v / S), nearest-even;
//     0x7F for a NaN sub-block;
//   * spread = kmax - kmin (0 without two active sub-blocks); spread <= 14
//     makes every v / S an E4M3 value, so the block converts exactly.
// v / S = e2m1 * 2^(k - kmax + 6) is formed exactly by decoding the E2M1 codes
// with the scale code k - kmax + 133 (clamped to [0, 254]: outside that range
// the values are zeros, or tinier than half E4M3's smallest subnormal), then
// encoded with scale 1: the gfx950 conversions are exact and round to
// nearest-even.
//
// The same kernel runs the quantization-aware step from master weights
// (BF16 / FP32): each 1x32 sub-block is first cast to MXFP4 with the MX cast's
// rules (and optionally stored as such), then goes through the steps above.
//
// One workgroup of 4 waves owns a 128-row x 256-column tile: two FP8 blocks
// side by side. Thread t = 16 g + h holds rows 8g .. 8g+7 of half sub-block h
// (16 codes: 8 bytes in, 16 bytes out), so 16 lanes cover a row and every
// MXFP4 load and FP8 store instruction moves whole 128-byte lines (4 rows of
// 128 bytes in, 4 rows of 256 bytes out). The transposed copy is staged as
// [column][row] bytes in LDS: each thread's 8 rows of a column are one 8-byte
// slot, slot g of column c stored at slot g ^ (c / 16) (conflict-free for a
// quarter wave), and leaves as 128-byte runs of the [C][R] plane.
#include "mx_cast_impl.h"   // memory helpers (non-temporal loads and stores)
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kRqRows = 128;
constexpr int kRqCols = 256;
constexpr int kRqThreads = 256;
constexpr int kRqWaves = kRqThreads / 64;
constexpr uint32_t kRqShift = 133;            // 127 + 6
constexpr int kRqRowsPerThread = 8;

// 4x4 byte transpose: byte j of result i is byte i of a[j].
__device__ __forceinline__ void transpose4x4(const uint32_t* a, uint32_t* c) {
  const uint32_t t0 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Max of two packed 16-bit fields over the whole wave.
__device__ __forceinline__ uint32_t wave_pk_max(uint32_t v) {
  v = pk_max_u16(v, dpp<kDppXor1>(v));
  v = pk_max_u16(v, dpp<kDppXor2>(v));
  v = pk_max_u16(v, dpp<kDppHalfMirror>(v));
  v = pk_max_u16(v, dpp<kDppRor8>(v));
  return pk_max_xor32(pk_max_xor16(v));
}

// 16 E2M1 codes (8 bytes) decoded with scale code c and re-encoded as E4M3 (16 bytes).
__device__ __forceinline__ void e2m1x16_to_e4m3(const uint2& w, uint32_t c, uint32_t* out) {
  const float sc = scale_operand(c);
  const float one = scale_operand(127u);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t cw = d ? w.y : w.x;
    const float2v f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 0);
    const float2v f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 1);
    const float2v f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 2);
    const float2v f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, sc, 3);
    uint32_t lo = cvt2_f32<kE4M3, false>(0u, f0[0], f0[1], one);
    lo = cvt2_f32<kE4M3, true>(lo, f1[0], f1[1], one);
    uint32_t hi = cvt2_f32<kE4M3, false>(0u, f2[0], f2[1], one);
    hi = cvt2_f32<kE4M3, true>(hi, f3[0], f3[1], one);
    out[2 * d] = lo;
    out[2 * d + 1] = hi;
  }
}

// Row r of this thread's half sub-block from the master weights: 16 elements
// (c0 + 16 h ..) in NV 16-byte chunks, quantized to MXFP4 with the 1x32 rules
// of the MX cast (the block max is shared with lane h ^ 1, which holds the
// other 16 elements). Returns the 8 code bytes and the E8M0 code.
template <bool BF16, int M>
__device__ __forceinline__ uint2 quantize16(const uint4* v, uint32_t& code) {
  uint2 w;
  if constexpr (BF16) {
    const uint32_t hm = pk_max_u16(pk_max_u16(pk_max_u16(v[0].x & 0x7FFF7FFFu, v[0].y & 0x7FFF7FFFu),
                                              pk_max_u16(v[0].z & 0x7FFF7FFFu, v[0].w & 0x7FFF7FFFu)),
                                   pk_max_u16(pk_max_u16(v[1].x & 0x7FFF7FFFu, v[1].y & 0x7FFF7FFFu),
                                              pk_max_u16(v[1].z & 0x7FFF7FFFu, v[1].w & 0x7FFF7FFFu)));
    uint32_t m = max(hm & 0xFFFFu, hm >> 16);
    m = max(m, dpp<kDppXor1>(m));
    code = scale_code<kE2M1, M, true>(m);
    w.x = encode8_bf16<kE2M1, M>(v[0].x, v[0].y, v[0].z, v[0].w, code).x;
    w.y = encode8_bf16<kE2M1, M>(v[1].x, v[1].y, v[1].z, v[1].w, code).x;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m = max(m, max(max(v[j].x & 0x7FFFFFFFu, v[j].y & 0x7FFFFFFFu), max(v[j].z & 0x7FFFFFFFu, v[j].w & 0x7FFFFFFFu)));
    m = max(m, dpp<kDppXor1>(m));
    code = scale_code<kE2M1, M, false>(m);
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c[j] = encode4_f32<kE2M1, M>(__uint_as_float(v[j].x), __uint_as_float(v[j].y), __uint_as_float(v[j].z),
                                   __uint_as_float(v[j].w), code);
    w = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
  }
  return w;
}

// SRC: kFromMx (an MXFP4 plane), kFromBf16 / kFromF32 (master weights, cast to
// MXFP4 first with scale rule M and, when asked, written out as such).
template <int SRC, int M, bool ROWS, bool COLS>
__global__ __launch_bounds__(kRqThreads) void requant_kernel(RqArgs a) {
  __shared__ uint32_t part[kRqWaves][2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[COLS ? kRqCols * kRqRows : 16];
  // the tile's 128 x 8 scale bytes, loaded as one dword per thread (kRqScaleWords)
  __shared__ __attribute__((aligned(4))) uint8_t lds_k[SRC == kFromMx ? kRqRows * 8 : 4];

  uint32_t bi, tr, tc;
  if (a.flags & kRqXcdRows) {
    // workgroup w runs on XCD w % 8: XCD x walks tile rows x, x + 8, ..., all
    // tile columns of each before the next (batch * tiles_r % 8 == 0)
    const uint32_t xcd = blockIdx.x % 8u, idx = blockIdx.x / 8u;
    const uint32_t rowi = (idx / a.tiles_c) * 8u + xcd;
    tc = idx % a.tiles_c;
    bi = rowi / a.tiles_r;
    tr = rowi - bi * a.tiles_r;
  } else {
    const uint32_t per_slice = a.tiles_r * a.tiles_c;
    bi = blockIdx.x / per_slice;
    const uint32_t rem = blockIdx.x % per_slice;
    tr = rem / a.tiles_c;
    tc = rem % a.tiles_c;
  }
  const int64_t R = a.rows, C = a.cols;
  const int64_t r0 = int64_t(tr) * kRqRows, c0 = int64_t(tc) * kRqCols;
  const int rows_in = int(min<int64_t>(R - r0, kRqRows));
  const int cols_in = int(min<int64_t>(C - c0, kRqCols));
  const uint32_t Cu = uint32_t(C);

  const int t = threadIdx.x;
  const int g = t >> 4, h = t & 15;
  const int sbk = h >> 1, blk = h >> 3;          // sub-block of the tile row, FP8 block
  const bool col_ok = 32 * sbk < cols_in;

  // ---- 8 rows x 16 codes (8 bytes) and their scales: loaded, or cast from the weights ----
  const int64_t tile_row = int64_t(bi) * R + r0;
  uint2 w[kRqRowsPerThread];
  uint32_t k[kRqRowsPerThread];
  if constexpr (SRC == kFromMx) {
    // tile origins (always inside the tensor); a lane outside it reads the origin instead
    const uint8_t* ct = a.codes + tile_row * (C / 2) + c0 / 2;
    const uint8_t* st = a.scales + tile_row * (C / 32) + c0 / 32;
    if (a.flags & kRqScaleWords) {
#pragma unroll
      for (int i = 0; i < kRqRowsPerThread; ++i) {
        const int row = kRqRowsPerThread * g + i;
        const bool ok = col_ok && row < rows_in;
        const u32x2 d = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(ct + (ok ? uint32_t(row) * (Cu / 2) + 8u * h : 0u)));
        w[i] = ok ? make_uint2(d.x, d.y) : make_uint2(0u, 0u);
      }
      // full-width tiles: thread t brings dword t & 1 of tile row t / 2's 8 scale
      // bytes into LDS (one load instead of 8 byte loads per thread)
      const int srow = t >> 1;
      const uint32_t kw = srow < rows_in
                              ? *reinterpret_cast<const uint32_t*>(st + uint32_t(srow) * (Cu / 32) + 4u * uint32_t(t & 1))
                              : 0u;
      reinterpret_cast<uint32_t*>(lds_k)[t] = kw;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kRqRowsPerThread; ++i) {
        const int row = kRqRowsPerThread * g + i;
        k[i] = (col_ok && row < rows_in) ? uint32_t(lds_k[row * 8 + sbk]) : 0u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRqRowsPerThread; ++i) {
        const int row = kRqRowsPerThread * g + i;
        const bool ok = col_ok && row < rows_in;
        const u32x2 d = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(ct + (ok ? uint32_t(row) * (Cu / 2) + 8u * h : 0u)));
        const uint32_t kk = st[ok ? uint32_t(row) * (Cu / 32) + sbk : 0u];
        w[i] = ok ? make_uint2(d.x, d.y) : make_uint2(0u, 0u);
        k[i] = ok ? kk : 0u;
      }
    }
  } else {
    constexpr bool BF16 = SRC == kFromBf16;
    constexpr uint32_t ES = BF16 ? 2 : 4;
    const uint8_t* xt = reinterpret_cast<const uint8_t*>(a.x) + (tile_row * C + c0) * ES;   // tile origin
    uint8_t* oc = a.out_codes ? a.out_codes + tile_row * (C / 2) + c0 / 2 + 8 * h : nullptr;
    uint8_t* os = a.out_scales ? a.out_scales + tile_row * (C / 32) + c0 / 32 + sbk : nullptr;
    // every row's loads are issued before the first is used. They are ordinary
    // (cache-allocating) loads: each instruction takes 16-byte pieces at a 32-
    // or 64-byte stride, and a line must stay in L2 until the 2 or 4 loads that
    // share it have run (non-temporal loads: 100 us instead of 78 us for
    // 14336 x 4096 FP32)
    constexpr int NV = BF16 ? 2 : 4;
    uint4 raw[kRqRowsPerThread][NV];
#pragma unroll
    for (int i = 0; i < kRqRowsPerThread; ++i) {
      const int row = kRqRowsPerThread * g + i;
      const bool ok = col_ok && row < rows_in;
      const uint8_t* p = xt + (ok ? (uint32_t(row) * Cu + 16u * h) * ES : 0u);
#pragma unroll
      for (int j = 0; j < NV; ++j) raw[i][j] = *reinterpret_cast<const uint4*>(p + 16 * j);
    }
#pragma unroll
    for (int i = 0; i < kRqRowsPerThread; ++i) {
      const int row = kRqRowsPerThread * g + i;
      const bool ok = col_ok && row < rows_in;
      if (!ok) {
#pragma unroll
        for (int j = 0; j < NV; ++j) raw[i][j] = make_uint4(0u, 0u, 0u, 0u);
      }
      uint32_t code;
      const uint2 c = quantize16<BF16, M>(raw[i], code);
      w[i] = ok ? c : make_uint2(0u, 0u);
      k[i] = ok ? code : 0u;
      if (ok && oc) *reinterpret_cast<uint2*>(oc + uint32_t(row) * (Cu / 2)) = c;
      if (ok && os && (h & 1) == 0) os[uint32_t(row) * (Cu / 32)] = uint8_t(code);
    }
  }

  // ---- kmax / kmin over active sub-blocks, per FP8 block (16-bit fields: k + 1, 256 - k) ----
  uint32_t nz = 0;                               // bit i: row i's half has a nonzero magnitude
#pragma unroll
  for (int i = 0; i < kRqRowsPerThread; ++i) nz |= (((w[i].x | w[i].y) & 0x77777777u) != 0u) ? 1u << i : 0u;
  nz |= dpp<kDppXor1>(nz);                       // the other half of the sub-block (lane h ^ 1)
  uint32_t fmax = 0, fmin = 0;
#pragma unroll
  for (int i = 0; i < kRqRowsPerThread; ++i) {
    const bool act = k[i] != 0xFFu && ((nz >> i) & 1u);
    fmax = max(fmax, act ? k[i] + 1u : 0u);
    fmin = max(fmin, act ? 256u - k[i] : 0u);
  }
  uint32_t pmax = wave_pk_max(blk ? fmax << 16 : fmax);
  uint32_t pmin = wave_pk_max(blk ? fmin << 16 : fmin);
  if ((t & 63) == 0) {
    part[t >> 6][0] = pmax;
    part[t >> 6][1] = pmin;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < kRqWaves; ++v) {
    pmax = pk_max_u16(pmax, part[v][0]);
    pmin = pk_max_u16(pmin, part[v][1]);
  }
  const uint32_t fa = blk ? pmax >> 16 : pmax & 0xFFFFu;
  const uint32_t fb = blk ? pmin >> 16 : pmin & 0xFFFFu;
  const int kmax = fa ? int(fa) - 1 : int(kRqShift);

  // ---- block scales and spreads (threads 0 and 8: the two blocks' first half sub-blocks) ----
  if (g == 0 && (h & 7) == 0 && col_ok) {
    const int64_t nbr = (R + kRqRows - 1) / kRqRows, nbc = (C + 127) / 128;
    const int64_t br = tr, bc = int64_t(2) * tc + blk;
    // 2^(kmax - 133): normal for kmax >= 7, subnormal below
    const uint32_t sbits = kmax >= 7 ? uint32_t(kmax - 6) << 23 : 1u << (kmax + 16);
    if (ROWS) a.block_scale[(int64_t(bi) * nbr + br) * nbc + bc] = __uint_as_float(sbits);
    if (COLS) a.block_scale_t[(int64_t(bi) * nbc + bc) * nbr + br] = __uint_as_float(sbits);
    if (a.spread) a.spread[(int64_t(bi) * nbr + br) * nbc + bc] = uint8_t(fa ? kmax - (256 - int(fb)) : 0);
  }

  // ---- convert: 16 codes per row -> 16 E4M3 bytes ----
  uint32_t e[kRqRowsPerThread][4];
#pragma unroll
  for (int i = 0; i < kRqRowsPerThread; ++i) {
    int c = int(k[i]) - kmax + int(kRqShift);
    c = c < 0 ? 0 : (c > 254 ? 254 : c);
    e2m1x16_to_e4m3(w[i], uint32_t(c), e[i]);
    if (k[i] == 0xFFu) e[i][0] = e[i][1] = e[i][2] = e[i][3] = 0x7F7F7F7Fu;
  }

  if constexpr (ROWS) {
    uint8_t* ot = a.fp8 + tile_row * C + c0 + 16 * h;
#pragma unroll
    for (int i = 0; i < kRqRowsPerThread; ++i) {
      const int row = kRqRowsPerThread * g + i;
      if (col_ok && row < rows_in)
        store_nt16(ot + uint32_t(row) * Cu, make_uint4(e[i][0], e[i][1], e[i][2], e[i][3]));
    }
  }

  if constexpr (COLS) {
    // column cl = 16 h + j: rows 8g .. 8g+7 as one 8-byte slot
    if (col_ok) {
      const int slot = (g ^ h) << 3;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo4[4] = {e[0][m], e[1][m], e[2][m], e[3][m]};
        const uint32_t hi4[4] = {e[4][m], e[5][m], e[6][m], e[7][m]};
        uint32_t lo[4], hi[4];
        transpose4x4(lo4, lo);
        transpose4x4(hi4, hi);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int cl = 16 * h + 4 * m + jj;
          *reinterpret_cast<uint2*>(lds_t + cl * kRqRows + slot) = make_uint2(lo[jj], hi[jj]);
        }
      }
    }
    __syncthreads();
    const uint32_t Ru = uint32_t(R);
    uint8_t* ot = a.fp8_t + (int64_t(bi) * C + c0) * R + r0;
#pragma unroll
    for (int i = 0; i < kRqCols * (kRqRows / 16) / kRqThreads; ++i) {
      const int id = t + i * kRqThreads;
      const int cl = id >> 3, c16 = id & 7;
      if (cl < cols_in && 16 * c16 < rows_in) {
        // logical slots 2 c16 and 2 c16 + 1 sit in one 16-byte chunk, swapped when cl / 16 is odd
        const int hh = (cl >> 4) & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(lds_t + cl * kRqRows + ((((2 * c16) ^ hh) >> 1) << 4));
        store_nt16(ot + uint32_t(cl) * Ru + 16u * c16, (hh & 1) ? make_uint4(v.z, v.w, v.x, v.y) : v);
      }
    }
  }
}

template <int SRC, int M, bool ROWS, bool COLS>
hipError_t launch_rq(const RqArgs& a, uint32_t nblocks, hipStream_t s) {
  return launch_kernel(requant_kernel<SRC, M, ROWS, COLS>, dim3(nblocks), dim3(kRqThreads), s, a);
}

template <int SRC, int M>
hipError_t launch_rq_axis(int axis, const RqArgs& a, uint32_t nblocks, hipStream_t s) {
  switch (axis) {
    case kRow: return launch_rq<SRC, M, true, false>(a, nblocks, s);
    case kCol: return launch_rq<SRC, M, false, true>(a, nblocks, s);
    default: return launch_rq<SRC, M, true, true>(a, nblocks, s);
  }
}

}  // namespace

hipError_t launch_requant(int src, int mode, int axis, const RqArgs& a, hipStream_t s) {
  const uint32_t nblocks = a.total_tiles;
  if (src == kFromMx) return launch_rq_axis<kFromMx, kFloor>(axis, a, nblocks, s);
  if (src == kFromBf16)
    return mode == kRoundUp ? launch_rq_axis<kFromBf16, kRoundUp>(axis, a, nblocks, s)
                            : launch_rq_axis<kFromBf16, kFloor>(axis, a, nblocks, s);
  return mode == kRoundUp ? launch_rq_axis<kFromF32, kRoundUp>(axis, a, nblocks, s)
                          : launch_rq_axis<kFromF32, kFloor>(axis, a, nblocks, s);
}

}  // namespace mx
