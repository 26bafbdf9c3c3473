// NVFP4 cast and dequantization.
//
// "MXFP4 と NVFP4 は何が違うのか調べてみた" §3, the §4 table and §7: E2M1 elements
// (the same as MXFP4's) in blocks of 16, each block with an unsigned E4M3
// (UE4M3, largest value 448) scale, and one FP32 global scale per tensor equal
// to the tensor's largest magnitude over 6 * 448. Every scale step is one FP32
// operation with round-to-nearest-even (IEEE-correct division), in this order:
//   g = A / 2688                          (A: largest finite |x| of the batch slice)
//   t = (amax_b / 6) / g    -> UE4M3      (RNE, saturating at 448)
//   r_b = 1 / (s_b * g)                   (per block; the §4 table applies NVFP4's
//   q = x * r_b             -> E2M1        scales by multiplication; RNE, saturating at 6)
//   y = (e2m1 * s_b) * g                  (dequantization; the first product is exact)
// A block whose scale code is 0, or whose r_b is not finite, or every block
// when g == 0, stores codes 0; a block holding NaN or Inf stores the UE4M3 NaN
// code 0x7F and codes 0. Codes are packed as MXFP4's (element 2k in the low nibble);
// block scales are [B][R][C/16] and, for the column copy (the same cast of
// X^T), [B][C][R/16].
//
// g takes two launches and the cast: zero the caller's [B] FP32 array, then
// fold every workgroup's amax into it with one atomic max, as FP32 bits with
// the sign bit set (magnitudes order as unsigned integers, and the set sign
// marks a raw maximum). Each cast workgroup divides a marked value by 2688
// itself and writes g back, so any read sees either the mark or the same g.
// The cast reuses the MX tiled kernel's layout (128 x 256 tiles, 8 waves,
// LDS-staged column codes).
//
// The cast never divides per element and rarely per block:
//  * r_b depends only on the block's scale code, so each workgroup divides once
//    per code (256 entries in LDS, shared by the tile).
//  * The block code is first estimated as fp32(amax_b * k), k = fp32(fp32(1/6) *
//    fp32(1/g)). Every rounding in the exact and the estimated chain is relative
//    error at most 2^-24 while amax_b >= 2^-120 and 2^-125 <= g <= 2^100, so the
//    estimate is within 6 FP32 ulps of the exact t. E4M3 rounding is monotone:
//    when t - 16 ulps and t + 16 ulps round to the same code, that is the code
//    of the exact t. Otherwise, or outside those ranges, the block takes the
//    two IEEE divisions.
#include "mx_cast_impl.h"

namespace mx {

namespace {

constexpr float kE2m1Max = 6.0f;
constexpr float kNvGlobalDiv = 6.0f * 448.0f;      // 2688
constexpr float kRcp6 = 0x1.555556p-3f;            // fp32(1/6)
constexpr uint32_t kNvWindow = 16;                 // ulps each side of the estimate
constexpr uint32_t kNvTcap = 0x49800000u;          // 2^20: every t above 464 saturates alike
constexpr uint32_t kNvAmin = 0x03800000u;          // 2^-120: amax/6 stays a normal FP32

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
  float rcp;         // 1 / (s_b * g)
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

// The defining computation: E4M3 of fp32(fp32(amax / 6) / g), RNE, overflow
// (0x7F) stepped down to 448. amag: FP32 bits of the block's largest magnitude
// (>= 0x7F800000: NaN or Inf present).
__device__ __forceinline__ uint32_t nv_code_exact(uint32_t amag, float g) {
  if (amag >= 0x7F800000u) return 0x7Fu;
  if (g == 0.0f) return 0u;
  const float t = (__uint_as_float(amag) / kE2m1Max) / g;
  return fix_overflow<kE4M3>(cvt2_f32<kE4M3, false>(0u, t, 0.0f, scale_operand(127u))) & 0xFFu;
}

// The same code through the estimate, falling back to nv_code_exact.
__device__ __forceinline__ uint32_t nv_code(uint32_t amag, const NvScale& s) {
  const uint32_t tb = min(__float_as_uint(__uint_as_float(amag) * s.k), kNvTcap);
  const uint32_t lo = tb > kNvWindow ? tb - kNvWindow : 0u;
  const uint32_t w = cvt2_f32<kE4M3, false>(0u, __uint_as_float(lo), __uint_as_float(tb + kNvWindow),
                                            scale_operand(127u));
  const uint32_t c0 = min(w & 0xFFu, 0x7Eu), c1 = min((w >> 8) & 0xFFu, 0x7Eu);
  uint32_t c = c0;
  bool slow = !(s.fast && amag >= kNvAmin && c0 == c1);
  if (amag == 0u && s.fast) { c = 0u; slow = false; }
  if (amag >= 0x7F800000u) { c = 0x7Fu; slow = false; }
  if (slow) c = nv_code_exact(amag, s.g);
  return c;
}

// LDS table of 1 / fp32(s_c * g) for every scale byte c; NaN marks the codes
// whose blocks store codes 0 (c == 0, or the reciprocal is not finite).
constexpr int kNvTab = 256;
__device__ __forceinline__ void nv_fill_table(float* tab, float g) {
  const int c = threadIdx.x;
  if (c < kNvTab) {
    const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uint32_t(c), scale_operand(127u), false)[0];
    const float r = 1.0f / (s * g);
    tab[c] = (c == 0 || !(__builtin_fabsf(r) < __builtin_inff())) ? __builtin_nanf("") : r;
  }
}

__device__ __forceinline__ NvBlock nv_block(uint32_t amag, const NvScale& s, const float* tab) {
  NvBlock b;
  b.code = nv_code(amag, s);
  b.rcp = tab[b.code];
  b.zero = b.rcp != b.rcp;
  return b;
}

// Four FP32 values times the block's reciprocal -> four E2M1 codes in the low 16 bits.
__device__ __forceinline__ uint32_t nv_encode4(float f0, float f1, float f2, float f3, const NvBlock& b) {
  const float one = scale_operand(127u);
  uint32_t w = cvt2_fp4_f32<0>(0u, f0 * b.rcp, f1 * b.rcp, one);
  w = cvt2_fp4_f32<1>(w, f2 * b.rcp, f3 * b.rcp, one);
  return b.zero ? 0u : (w & 0xFFFFu);
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
  __shared__ __attribute__((aligned(4))) uint8_t lds_scales[COLS ? kTileC * SPC : 4];
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
  __shared__ __attribute__((aligned(16))) uint32_t lds_rs[ROWLDS ? kTileR * 4 : 4];
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

  const int wid = threadIdx.x >> 6;
  const int wr = wid % kWaveRows, wc = wid / kWaveRows;
  const int lane = threadIdx.x & 63;
  const int q = lane / LPR, t = lane % LPR;
  const int lcol = 128 * wc + t * VEC;
  const int lrow = 32 * wr + RPT * q;
  const bool col_ok = lcol < cols_in;

  const int64_t tile_elem = (int64_t(bi) * R + r0) * C + c0;
  const uint8_t* xt = reinterpret_cast<const uint8_t*>(a.x) + tile_elem * ES;
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
      for (int d = 0; d < 4; ++d) {
        cm[d] = pk_max_xor16(cm[d]);                     // row groups q and q ^ 1
        cb[2 * d] = nv_block((cm[d] & 0xFFFFu) << 16, sc, lds_rtab);
        cb[2 * d + 1] = nv_block(cm[d] & 0xFFFF0000u, sc, lds_rtab);
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
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      uint32_t m;
      if constexpr (BF16) {
        const uint32_t h = pk_max_u16(pk_max_u16(v[k].x & 0x7FFF7FFFu, v[k].y & 0x7FFF7FFFu),
                                      pk_max_u16(v[k].z & 0x7FFF7FFFu, v[k].w & 0x7FFF7FFFu));
        m = max(h & 0xFFFFu, h >> 16) << 16;
        m = max(m, dpp<kDppXor1>(m));
      } else {
        m = max(max(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu), max(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu));
        m = group_max<4>(m);
      }
      const NvBlock blk = nv_block(m, sc, lds_rtab);
      const bool ok = col_ok && lrow + k < rows_in;
      uint8_t* dst = rct + rcoff + uint32_t(k) * Cu / 2;
      if constexpr (BF16) {
        const uint32_t w = nv_encode4(elem(k, 0), elem(k, 1), elem(k, 2), elem(k, 3), blk) |
                           (nv_encode4(elem(k, 4), elem(k, 5), elem(k, 6), elem(k, 7), blk) << 16);
        if constexpr (ROWLDS) *reinterpret_cast<uint32_t*>(lds_rows + rows_off(lrow + k, lcol)) = w;
        else if (ok) store_nt4(dst, w);
      } else {
        const uint32_t w = nv_encode4(elem(k, 0), elem(k, 1), elem(k, 2), elem(k, 3), blk);
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
        if (t % HALF == 0) lds_rs[(lrow + k) * 4 + dcol / 64] = sb;
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
      const int off = cl * BPC + ((((byte0 >> 4) ^ ((cl >> 3) & (CPC - 1))) << 4) | (byte0 & 15));
      if constexpr (BF16) {
        const uint32_t w = nv_encode4(elem(0, j), elem(1, j), elem(2, j), elem(3, j), cb[j]) |
                           (nv_encode4(elem(4, j), elem(5, j), elem(6, j), elem(7, j), cb[j]) << 16);
        *reinterpret_cast<uint32_t*>(lds_codes + off) = w;               // 8 rows in 4 bytes
      } else {
        uint32_t w[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          w[g4] = nv_encode4(elem(4 * g4, j), elem(4 * g4 + 1, j), elem(4 * g4 + 2, j), elem(4 * g4 + 3, j), cb[j]);
        *reinterpret_cast<uint2*>(lds_codes + off) = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
      }
    }
    // column block index inside the tile: 16-row groups
    if (BF16 ? (q % 2 == 0) : true) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) lds_scales[(lcol + j) * SPC + lrow / 16] = uint8_t(cb[j].code);
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
        const uint4 w = *reinterpret_cast<const uint4*>(lds_codes + cl * BPC + ((part ^ ((cl >> 3) & (CPC - 1))) << 4));
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
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(lds_rs + rl * 4);
    }
    if (int(threadIdx.x) < cols_in) {
      const int cl = threadIdx.x;
      uint8_t* dst = a.col_scales + ctile_elem / 16 + uint32_t(cl) * Ru / 16;
      if ((a.flags & kColScaleDword) && rows_in == kTileR) {
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(lds_scales + cl * SPC);
        *reinterpret_cast<uint32_t*>(dst + 4) = *reinterpret_cast<const uint32_t*>(lds_scales + cl * SPC + 4);
      } else {
#pragma unroll
        for (int s = 0; s < SPC; ++s)
          if (16 * s < rows_in) dst[s] = lds_scales[cl * SPC + s];
      }
    }
  }
}

template <bool BF16, int AX>
hipError_t launch_nv_cast(const NvArgs& a, uint32_t nblocks, hipStream_t s) {
  hipLaunchKernelGGL((nv_cast_kernel<BF16, AX>), dim3(nblocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
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
  hipLaunchKernelGGL(nv_zero_kernel, dim3(small), dim3(256), 0, s, gb, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunks = slice_elems * (in_bf16 ? 2 : 4) / 16;
  const int64_t per_block = int64_t(kAmaxThreads) * kAmaxUnroll;
  const int64_t want = (chunks + per_block - 1) / per_block;
  const int64_t cap = batch >= kAmaxBlocks ? 1 : kAmaxBlocks / batch;
  const dim3 grid(uint32_t(want < cap ? want : cap), uint32_t(batch));
  if (in_bf16)
    hipLaunchKernelGGL(nv_amax_kernel<true>, grid, dim3(kAmaxThreads), 0, s, static_cast<const uint8_t*>(x), gb, chunks);
  else
    hipLaunchKernelGGL(nv_amax_kernel<false>, grid, dim3(kAmaxThreads), 0, s, static_cast<const uint8_t*>(x), gb, chunks);
  return hipGetLastError();
}

hipError_t launch_nvfp4_cast(bool in_bf16, int axis, const NvArgs& a, uint32_t nblocks, hipStream_t s) {
  return in_bf16 ? nv_by_axis<true>(axis, a, nblocks, s) : nv_by_axis<false>(axis, a, nblocks, s);
}

hipError_t launch_nvfp4_dequant(bool out_bf16, const uint8_t* codes, const uint8_t* scales, const float* gs,
                                void* y, int64_t nblocks, int64_t blocks_per_slice, hipStream_t s) {
  const uint32_t grid = uint32_t((nblocks + kDqThreads - 1) / kDqThreads);
  if (out_bf16)
    hipLaunchKernelGGL(nv_dequant_kernel<true>, dim3(grid), dim3(kDqThreads), 0, s, codes, scales, gs, y, nblocks,
                       blocks_per_slice);
  else
    hipLaunchKernelGGL(nv_dequant_kernel<false>, dim3(grid), dim3(kDqThreads), 0, s, codes, scales, gs, y, nblocks,
                       blocks_per_slice);
  return hipGetLastError();
}

}  // namespace mx
