// MX block quantization kernels: row-wise, column-wise and fused row+column,
// with round-to-nearest-even or stochastic rounding, and 1x32 or 32x32 blocks.
// This header holds the kernel templates; mx_cast.hip, mx_cast_2d.hip and
// mx_cast_sr.hip instantiate them (one translation unit per variant family).
//
// What is computed ("MXFP4 と NVFP4 は何が違うのか調べてみた" §2 and §4): every block
// of 32 elements gets one E8M0 scale 2^e chosen from the block's largest
// magnitude (OCP floor rule or the round-up rule), and each element is stored
// as x / 2^e in the element format with round-to-nearest-even and clipping at
// the format's largest value. Row blocks run along the contiguous axis;
// column blocks are 32 rows of one column and are written transposed, so the
// column copy is the row-wise quantization of X^T.
//
// Work decomposition (gfx950, 64-wide waves). A workgroup of 8 waves owns a
// 128-row x 256-column tile of one batch slice and reads it from HBM once (the
// FP32 column-only cast with stochastic rounding: 128 x 128, each wave 64
// columns wide, see kNarrow):
//   * wave w = 4 * wc + wr covers rows 32*wr .. +31 and columns 128*wc .. +127;
//     lane = q * LPR + t, where t picks a 16-byte chunk of a row (8 BF16 or
//     4 FP32 elements) and q a group of RPT consecutive rows. One wave thus
//     holds exactly one 32-row column block for each of its 128 columns.
//   * row blocks: lane-local max, then a max over the 4 (BF16) or 8 (FP32)
//     lanes sharing the block; codes go straight to HBM, and the 4 scale bytes
//     of a row's 128 columns are gathered into one dword store.
//   * column blocks: in-lane max over the thread's RPT rows, then a max over
//     the RG lanes holding the other rows of the block. The codes (1 byte, not
//     the inputs) are staged in LDS as [column][row] with a 16-byte XOR swizzle
//     and written out as runs of the transposed plane (128 bytes per column
//     for 8-bit codes; 6-bit codes are packed 16 -> 12 bytes on the way out).
// Memory-system choices, measured on MI355X with input and output buffers
// rotated through more memory than the 256 MB last-level cache holds: the
// input is read and both code planes are written with non-temporal accesses
// (6-bit code planes excepted: their runs do not fill whole 128-byte lines),
// while the scale planes go through L2 with ordinary stores (scale bytes of one
// 128-byte line come from several workgroups and must merge in L2; making them
// non-temporal costs 60%). Tiles are ordered so that each XCD owns a strip of
// adjacent tile columns and sweeps down the rows.
#pragma once
#include "mx_device.h"
#include "mx_kernels.h"
#include "mx_sr.h"

namespace mx {

namespace {

constexpr int kXcds = 8;                     // tile geometry: mx_enums.h

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt4(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
// Three dword stores to consecutive addresses; the compiler merges them into
// one 12-byte store (global_store_dwordx3), which needs only 4-byte alignment.
__device__ __forceinline__ void store_nt12(void* p, uint32_t a, uint32_t b, uint32_t c) {
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  __builtin_nontemporal_store(a, q);
  __builtin_nontemporal_store(b, q + 1);
  __builtin_nontemporal_store(c, q + 2);
}
// The same through L2 with ordinary stores. A tile's 6-bit code runs are 96 or
// 192 bytes long, so 128-byte lines are shared by neighbouring tiles (which the
// tile order keeps on one XCD at about the same time); ordinary stores let
// those partial lines merge in L2 before they are written back. Non-temporal
// partial lines made the fused FP6 cast 36% slower on MI355X.
__device__ __forceinline__ void store12(void* p, uint32_t a, uint32_t b, uint32_t c) {
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  q[0] = a;
  q[1] = b;
  q[2] = c;
}
// A dword store with the agent-scope bit (sc1). Used for the row-scale plane of
// the 6-bit formats, whose ordinary code stores keep L2 full of dirty partial
// lines: there it measured 1.5-3% faster on MI355X than a plain store. With the
// non-temporal code planes of the other formats it measured 6% slower. (A 4-byte
// store has no data hazard with the next VALU write, so no wait state is due.)
__device__ __forceinline__ void store_sc1_4(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
// The same for 8 bytes (still no wait state due: the data hazard needs more than 8).
__device__ __forceinline__ void store_sc1_8(void* p, uint32_t lo, uint32_t hi) {
  const u32x2 d = u32x2{lo, hi};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(d) : "memory");
}
__device__ __forceinline__ void store_nt2(void* p, uint32_t v) {
  __builtin_nontemporal_store(static_cast<unsigned short>(v), reinterpret_cast<unsigned short*>(p));
}

// Buffer stores. A tile's stores to one plane go through a descriptor whose base is the
// same for the whole wave (the tile's, or the wave's, first byte of that plane) and whose
// range covers every byte the tile may write there. A lane with nothing to write passes
// kOutOfRange, which lies past every range used here (all below 2^31 bytes, from the
// host's limits C < 2^22 and R < 2^23), and the hardware drops its store. The stores then
// need no branches, and 32-bit offsets replace 64-bit addresses: in the fused 8-bit cast
// that took 117 VGPRs to 89 and 48.68 us to 48.47 (16384 x 4096 BF16, MI355X).
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufNt = 2;                    // cache-policy operand of a non-temporal access
typedef unsigned int bu32x2 __attribute__((__vector_size__(8)));
typedef unsigned int bu32x4 __attribute__((__vector_size__(16)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(void* base, uint32_t bytes) {
  // word 3 selects the 32-bit data format that untyped buffer accesses expect on gfx9-family GPUs
  return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void bstore_nt16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(bu32x4{v.x, v.y, v.z, v.w}, r, off, 0, kBufNt);
}
__device__ __forceinline__ void bstore_nt8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(bu32x2{v.x, v.y}, r, off, 0, kBufNt);
}
__device__ __forceinline__ void bstore_nt4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kBufNt);
}
__device__ __forceinline__ void bstore_nt2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v), r, off, 0, kBufNt);
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(bu32x2{v.x, v.y}, r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// Workgroup i runs on XCD i % 8. Give XCD x the x-th contiguous eighth of a
// tile sequence that is ordered strip-major: tile columns are cut into 8
// strips, and each strip is walked batch by batch, row by row. Neighbouring
// tiles of one strip then run at the same time on the same XCD.
//
// stagger: strip s starts its walk s * (rows_total / 16) tile rows further
// down (wrapping). All strips advance at about the same pace, so without it
// every column-plane store in flight lands in the same few KiB of its
// transposed row; when that row's pitch is a multiple of 4 KiB those stores
// share address bits and crowd a subset of the HBM channels. The rotation is
// a permutation of each strip's tiles, so every tile is still visited once.
__device__ __forceinline__ void tile_coords(uint32_t bid, uint32_t nb, uint32_t tiles_r, uint32_t tiles_c,
                                            bool stagger, uint32_t& b, uint32_t& tr, uint32_t& tc) {
  const uint32_t xcd = bid % kXcds, idx = bid / kXcds;
  const uint32_t per = nb / kXcds, rem = nb % kXcds;
  const uint32_t i = xcd * per + min(xcd, rem) + idx;                // position in the sequence
  const uint32_t w = (tiles_c + kXcds - 1) / kXcds;                  // strip width in tiles
  const uint32_t rows_total = nb / tiles_c;                          // batch * tiles_r
  const uint32_t strip = i / (rows_total * w);
  const uint32_t in = i - strip * rows_total * w;
  const uint32_t ws = min(w, tiles_c - strip * w);
  const uint32_t rowi0 = in / ws;
  tc = strip * w + (in - rowi0 * ws);
  // strip <= 7, so the rotated index stays below 2 * rows_total
  const uint32_t rot = rowi0 + (stagger ? strip * max(1u, rows_total / 16u) : 0u);
  const uint32_t rowi = rot >= rows_total ? rot - rows_total : rot;
  b = rowi / tiles_r;
  tr = rowi - b * tiles_r;
}

// RD: kRne or kSr (stochastic rounding, mx_sr.h). B2: one scale per 32x32
// block (the wave's 32 rows x 32 columns) instead of per 1x32 block; the
// column copy then shares the block's scale, and the scale planes are the
// [R/32][C/32] grid and its transpose.
//
// The FP32 column-only cast with stochastic rounding uses narrow tiles (kNarrow
// below): 128 x 128, each wave 32 rows x 64 columns, so a lane holds 8 rows of
// 4 elements instead of 16. Its Philox draws and their decisions then fit two
// workgroups per CU (at most 128 VGPRs) instead of one.
template <bool BF16, int F, int M, int AX, int RD, bool B2>
constexpr bool kNarrow = RD == kSr && !BF16 && AX == kCol && !B2;

template <bool BF16, int F, int M, int AX, int RD, bool B2>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    kNarrow<BF16, F, M, AX, RD, B2> ? 4 : (RD == kSr ? 2 : (BF16 ? 4 : (AX == kBoth ? 2 : 3)))))) void
mx_cast_kernel(CastArgs a) {
  constexpr int VEC = InC<BF16>::vec;          // elements per 16-byte chunk
  constexpr int ES = BF16 ? 2 : 4;             // input element bytes
  constexpr bool NARROW = kNarrow<BF16, F, M, AX, RD, B2>;
  constexpr int TC = NARROW ? kTileCNarrow : kTileC;   // tile columns: 256 | 128
  constexpr int WCS = TC / kWaveCols;          // columns per wave: 128 | 64
  constexpr int LPR = WCS / VEC;               // lanes per wave row: 16 | 32 (narrow FP32: 16)
  constexpr int RG = 64 / LPR;                 // row groups per wave: 4 | 2
  constexpr int RPT = 32 / RG;                 // rows per thread: 8 | 16
  constexpr int LPB = 32 / VEC;                // lanes per row block: 4 | 8
  constexpr int CB = FmtC<F>::bits;            // code bits in memory: 8 | 6 | 4
  constexpr int RB = kRegBits<F>;              // code bits as formed and staged: 8 | 4
  constexpr bool ROWS = (AX & kRow) != 0;
  constexpr bool COLS = (AX & kCol) != 0;
  constexpr int BPC = kTileR * RB / 8;         // staged code bytes per tile column: 128 | 64
  constexpr int CPC = BPC / 16;                // 16-byte chunks per staged column: 8 | 4
  constexpr bool CM = COLS || B2;              // column maxima needed
  constexpr bool SR = RD == kSr;
  // stochastic rounding through the fast path, except in the FP32 row+column
  // kernel, where the extra registers would spill
  constexpr bool SRFAST = !(AX == kBoth && !BF16);

  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[COLS ? TC * BPC : 16];
  // column-block scale codes as [wave row][tile column]: a lane's codes of its VEC
  // columns are contiguous and leave in one store
  __shared__ __attribute__((aligned(8))) uint8_t lds_scales[COLS ? TC * kWaveRows : 8];
  // 4-bit codes with both copies: a wave row's row codes are only 64 bytes, half
  // of a 128-byte line whose other half comes from the neighbouring wave. They are
  // staged here as [tile row][128 bytes] and, after the barrier the column copy
  // needs anyway, written out as whole lines.
  constexpr bool ROWLDS = ROWS && COLS && CB == 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_rows[ROWLDS ? kTileR * kTileC / 2 : 16];
  // byte offset of (tile row r, tile column c) in lds_rows: the 16-byte chunk index
  // XORed with (r / 8) mod 8, so that the 4 row groups of a wave hit different banks
  auto rows_off = [](int r, int c) { return r * (kTileC / 2) + ((c / 2) ^ (((r >> 3) & 7) << 4)); };
  // 6-bit codes from BF16 with both copies: a wave row's 96 bytes, stored 12 at
  // a time by half the lanes, straddle lines. They are staged as [tile row][192
  // bytes] (row pitch padded by 16 bytes against bank conflicts between row
  // groups) and written as 16-byte chunks, all lanes busy, when the row-plane
  // pitch 3C/4 is a multiple of 16 bytes (cols % 64 == 0); otherwise directly.
  // (The FP32 kernel, at one workgroup per CU, measured slower staged.)
  constexpr bool ROWLDS6 = ROWS && COLS && CB == 6 && BF16;
  constexpr int P6 = kTileC * 6 / 8 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds_rows6[ROWLDS6 ? kTileR * P6 : 16];
  // Row scales with both copies and full-width tiles (kRowScaleQword: cols % 256
  // == 0, plane 8-byte aligned): the two waves' scale dwords of a tile row are
  // staged and leave as one 8-byte store after the barrier. That halves the
  // stores, and each tile's piece of a 128-byte scale line arrives in one
  // transaction. Such a line is written by all 8 XCDs.
  constexpr bool RS8 = ROWS && COLS && !B2;
  __shared__ uint32_t lds_rs[RS8 ? kTileR * 2 : 1];

  uint32_t bi, tr, tcol;
  tile_coords(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_c, (a.flags & kStaggerStrips) != 0, bi, tr, tcol);
  const int64_t R = a.rows, C = a.cols;
  const int64_t r0 = int64_t(tr) * kTileR;
  const int64_t c0 = int64_t(tcol) * TC;
  // rows / columns of this tile inside the tensor (ragged last tiles)
  const int rows_in = int(min<int64_t>(R - r0, kTileR));
  const int cols_in = int(min<int64_t>(C - c0, TC));
  const uint32_t Cu = uint32_t(C);             // host guarantees C < 2^22 and, for columns, R < 2^23
  const bool lines6 = ROWLDS6 && (Cu & 63u) == 0u;
  const bool rs8 = RS8 && (a.flags & kRowScaleQword) != 0;

  const int wid = threadIdx.x >> 6;
  const int wr = wid % kWaveRows, wc = wid / kWaveRows;
  const int lane = threadIdx.x & 63;
  const int q = lane / LPR, t = lane % LPR;
  const int lcol = WCS * wc + t * VEC;                    // column inside the tile
  const int lrow = 32 * wr + RPT * q;                     // first row of this thread inside the tile
  const bool col_ok = lcol < cols_in;

  // tile origins (uniform across the workgroup) and 32-bit per-thread offsets
  const int64_t tile_elem = (int64_t(bi) * R + r0) * C + c0;
  const uint8_t* xt = reinterpret_cast<const uint8_t*>(a.x) + tile_elem * ES;
  const uint32_t xoff = (uint32_t(lrow) * Cu + uint32_t(lcol)) * ES;
  // Every lane loads (lanes outside a ragged tile read the tile origin, which
  // always exists, and then zero their data), so the 8 or 16 loads issue back
  // to back without branches between them.
  uint4 v[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const bool ok = col_ok && lrow + k < rows_in;
    const uint4 d = load_nt(xt + (ok ? xoff + uint32_t(k) * Cu * ES : 0u));
    v[k] = ok ? d : make_uint4(0u, 0u, 0u, 0u);
  }

  // Stochastic rounding: the draws of this thread's VEC elements of row k
  // (flat element index (bi*R + row)*C + column; 8 consecutive elements share
  // one Philox block, so an FP32 lane uses half of its block). BF16 keeps the
  // draws of all its rows in registers; FP32, with twice the rows, draws them
  // again where they are used.
  auto row_draws = [&](int k, uint32_t* out) {
    const int64_t i0 = tile_elem + int64_t(lrow + k) * C + lcol;
    const uint4 w = sr_words(uint64_t(i0) >> 3, a.seed_lo, a.seed_hi);
    if constexpr (BF16) {
      out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
    } else {
      const bool hi = (i0 & 4) != 0;                       // elements 4..7 of the block: words 2, 3
      out[0] = hi ? w.z : w.x;
      out[1] = hi ? w.w : w.y;
    }
  };
  // FP32: lanes t and t ^ 1 hold the two halves of each row's Philox block
  // (t even: elements 0..3, words 0 and 1). Lane t computes the block of row
  // k + (t & 1) and the pair swaps the halves the other needs (DPP), so each
  // block is generated once for two rows.
  auto row_draws_pair = [&](int k, uint32_t* d0, uint32_t* d1) {
    const int p = t & 1;
    const int64_t i0 = tile_elem + int64_t(lrow + k + p) * C + lcol;
    const uint4 w = sr_words(uint64_t(i0) >> 3, a.seed_lo, a.seed_hi);
    const uint32_t r0 = dpp<kDppXor1>(p ? w.x : w.z), r1 = dpp<kDppXor1>(p ? w.y : w.w);
    d0[0] = p ? r0 : w.x;
    d0[1] = p ? r1 : w.y;
    d1[0] = p ? w.z : r0;
    d1[1] = p ? w.w : r1;
  };
  constexpr bool KEEP = SR && BF16;
  uint32_t draw[KEEP ? RPT : 1][VEC / 2];
  if constexpr (KEEP) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) row_draws(k, draw[k]);
  }

  // Column-block maxima need every row this thread loaded, so they are formed
  // first: the loads are all consumed before the first store is issued, and no
  // wait on the vector-memory counter (which also counts stores) sits between
  // the stores below.
  uint32_t code_j[COLS ? VEC : 1];
  uint32_t code2d = 0;                         // B2: the scale code of this lane's 32x32 block
  if constexpr (CM) {
    uint32_t cm[4];
    if constexpr (BF16) {
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = (&v[0].x)[d] & 0x7FFF7FFFu;
#pragma unroll
      for (int k = 1; k < RPT; ++k) {
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], (&v[k].x)[d] & 0x7FFF7FFFu);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = pk_max_xor32(pk_max_xor16(cm[d]));   // the 4 row groups
      if constexpr (B2) {
        const uint32_t h = pk_max_u16(pk_max_u16(cm[0], cm[1]), pk_max_u16(cm[2], cm[3]));
        code2d = scale_code<F, M, true>(group_max<LPB>(max(h & 0xFFFFu, h >> 16)));
      }
      if constexpr (COLS) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          code_j[2 * d] = B2 ? code2d : scale_code<F, M, true>(cm[d] & 0xFFFFu);
          code_j[2 * d + 1] = B2 ? code2d : scale_code<F, M, true>(cm[d] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = (&v[0].x)[d] & 0x7FFFFFFFu;
#pragma unroll
      for (int k = 1; k < RPT; ++k) {
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = max(cm[d], (&v[k].x)[d] & 0x7FFFFFFFu);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {                           // the row groups of the 32-row block
        cm[d] = max_xor32(cm[d]);
        if constexpr (RG == 4) cm[d] = max_xor16(cm[d]);
      }
      if constexpr (B2) code2d = scale_code<F, M, false>(group_max<LPB>(max(max(cm[0], cm[1]), max(cm[2], cm[3]))));
      if constexpr (COLS) {
#pragma unroll
        for (int d = 0; d < 4; ++d) code_j[d] = B2 ? code2d : scale_code<F, M, false>(cm[d]);
      }
    }
  }

  // ---------------- row-wise blocks ----------------
  if constexpr (ROWS) {
    uint8_t* rct = reinterpret_cast<uint8_t*>(a.row_codes) + tile_elem * CB / 8;
    const uint32_t rcoff = (uint32_t(lrow) * Cu + uint32_t(lcol)) * CB / 8;
    // the tile's 128 rows of the row plane (below 2^29 bytes). The row-only tiled kernel
    // (32x32 blocks) keeps plain stores: there the per-row offsets would raise its light
    // register use (FP32: 77 -> 99 VGPRs, three workgroups per CU -> two).
    const __amdgpu_buffer_rsrc_t rc_rsrc = plane_rsrc(rct, uint32_t(kTileR) * Cu * CB / 8);
    uint32_t scale_dw = 0;                      // 4 scale bytes of one row's 128 wave columns, lane t == k
    uint32_t dk_even[VEC / 2], dk_odd[VEC / 2];   // FP32 with SR: the draws of rows k and k + 1 (k even)
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      uint32_t m;
      if constexpr (BF16) {
        const uint32_t h = pk_max_u16(pk_max_u16(v[k].x & 0x7FFF7FFFu, v[k].y & 0x7FFF7FFFu),
                                      pk_max_u16(v[k].z & 0x7FFF7FFFu, v[k].w & 0x7FFF7FFFu));
        m = max(h & 0xFFFFu, h >> 16);
      } else {
        m = max(max(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu), max(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu));
      }
      m = group_max<LPB>(m);
      const uint32_t code = B2 ? code2d : scale_code<F, M, BF16>(m);
      const bool ok = col_ok && lrow + k < rows_in;
      uint8_t* dst = rct + rcoff + uint32_t(k) * Cu * CB / 8;
      const uint32_t rc_off = ok ? rcoff + uint32_t(k) * Cu * CB / 8 : kOutOfRange;
      if constexpr (BF16) {
        const uint2 w = SR ? encode8_sr<true, F, M, SRFAST>(v[k], draw[KEEP ? k : 0], code)
                           : encode8_bf16<F, M>(v[k].x, v[k].y, v[k].z, v[k].w, code);
        if constexpr (CB == 6) {
          // 48 bits per lane: even lanes store theirs and the odd neighbour's as 12 bytes
          const uint32_t hi = pack6(w.y);
          const uint32_t e0 = pack6(w.x) | (hi << 24), e1 = hi >> 8;
          const uint32_t o0 = dpp<kDppXor1>(e0), o1 = dpp<kDppXor1>(e1);
          if (lines6) {
            if ((t & 1) == 0) {
              uint32_t* l = reinterpret_cast<uint32_t*>(lds_rows6 + (lrow + k) * P6 + (96 * wc + 6 * t));
              l[0] = e0;
              l[1] = e1 | (o0 << 16);
              l[2] = (o0 >> 16) | (o1 << 16);
            }
          } else if (ok && (t & 1) == 0) {
            store12(dst, e0, e1 | (o0 << 16), (o0 >> 16) | (o1 << 16));
          }
        } else if constexpr (ROWLDS) {
          *reinterpret_cast<uint32_t*>(lds_rows + rows_off(lrow + k, lcol)) = w.x;
        } else if constexpr (!COLS) {
          if (ok) {
            if constexpr (CB == 8) store_nt8(dst, w);
            else store_nt4(dst, w.x);
          }
        } else if constexpr (CB == 8) {
          bstore_nt8(rc_rsrc, rc_off, w);
        } else {
          bstore_nt4(rc_rsrc, rc_off, w.x);
        }
      } else {
        uint32_t w;
        if constexpr (SR) {
          if ((k & 1) == 0) row_draws_pair(k, dk_even, dk_odd);
          w = encode8_sr<false, F, M, SRFAST>(v[k], (k & 1) ? dk_odd : dk_even, code).x;
        } else {
          w = encode4_f32<F, M>(__uint_as_float(v[k].x), __uint_as_float(v[k].y), __uint_as_float(v[k].z),
                                __uint_as_float(v[k].w), code);
        }
        if constexpr (CB == 6) {
          // 24 bits per lane: lane 4i stores the 12 bytes of lanes 4i .. 4i+3
          const uint32_t g0 = pack6(w);
          const uint32_t g1 = dpp<kDppQuadNext>(g0), g2 = dpp<kDppXor2>(g0), g3 = dpp<kDppQuadPrev>(g0);
          if (lines6) {
            if ((t & 3) == 0) {
              uint32_t* l = reinterpret_cast<uint32_t*>(lds_rows6 + (lrow + k) * P6 + (96 * wc + 3 * t));
              l[0] = g0 | (g1 << 24);
              l[1] = (g1 >> 8) | (g2 << 16);
              l[2] = (g2 >> 16) | (g3 << 8);
            }
          } else if (ok && (t & 3) == 0) {
            store12(dst, g0 | (g1 << 24), (g1 >> 8) | (g2 << 16), (g2 >> 16) | (g3 << 8));
          }
        } else if constexpr (ROWLDS) {
          *reinterpret_cast<uint16_t*>(lds_rows + rows_off(lrow + k, lcol)) = uint16_t(w);
        } else if constexpr (!COLS) {
          if (ok) {
            if constexpr (CB == 8) store_nt4(dst, w);
            else store_nt2(dst, w);
          }
        } else if constexpr (CB == 8) {
          bstore_nt4(rc_rsrc, rc_off, w);
        } else {
          bstore_nt2(rc_rsrc, rc_off, w);
        }
      }
      if constexpr (B2) continue;                 // one scale per 32x32 block, stored below
      // OR the 4 block codes of this wave row into one dword: lanes t, t^LPB, ..
      uint32_t sb = code << (8 * (t / LPB));
      if constexpr (BF16) {
        sb |= dpp<kDppRor4>(sb);
        sb |= dpp<kDppRor8>(sb);
      } else {
        sb |= dpp<kDppRor8>(sb);
        sb = or_xor16(sb);
      }
      scale_dw = (t == k) ? sb : scale_dw;
    }
    if constexpr (B2) {
      // the wave's 4 block scales, row (r0 + 32 wr) / 32 of the [R/32][C/32] grid
      uint32_t sb = code2d << (8 * (t / LPB));
      if constexpr (BF16) {
        sb |= dpp<kDppRor4>(sb);
        sb |= dpp<kDppRor8>(sb);
      } else {
        sb |= dpp<kDppRor8>(sb);
        sb = or_xor16(sb);
      }
      if (lane == 0 && 32 * wr < rows_in && 128 * wc < cols_in) {
        const int64_t nbc = C / 32;
        uint8_t* dst = a.row_scales + (int64_t(bi) * (R / 32) + (r0 / 32 + wr)) * nbc + (c0 + 128 * wc) / 32;
        if (a.flags & kRowScaleDword) {
          *reinterpret_cast<uint32_t*>(dst) = sb;
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (128 * wc + 32 * m < cols_in) dst[m] = uint8_t(sb >> (8 * m));
        }
      }
    }
    // lane t < RPT stores the scale bytes of tile row lrow + t, wave columns 128*wc .. +127
    // (or stages them for the 8-byte store after the barrier)
    if (rs8) {
      if (t < RPT) lds_rs[(lrow + t) * 2 + wc] = scale_dw;
    } else if (!B2 && t < RPT && lrow + t < rows_in && 128 * wc < cols_in) {
      uint8_t* dst = a.row_scales + tile_elem / 32 + (uint32_t(lrow + t) * Cu + uint32_t(128 * wc)) / 32;
      if (a.flags & kRowScaleDword) {
        if constexpr (CB == 6) store_sc1_4(dst, scale_dw);
        else *reinterpret_cast<uint32_t*>(dst) = scale_dw;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (128 * wc + 32 * m < cols_in) dst[m] = uint8_t(scale_dw >> (8 * m));
      }
    }
  }

  // ---------------- column-wise blocks ----------------
  if constexpr (COLS) {
    // encode column j of this thread (rows lrow .. +RPT-1) and stage it at
    // [column][row], the 16-byte chunk index XORed with (column / 8) mod CPC
    const int byte0 = lrow * RB / 8;                  // this thread's offset inside a staged column
    // With 8-byte staging writes (8 rows of 1-byte codes), the 16 lanes of a quarter-wave
    // write 16 columns, and columns 64 apart take the same chunk swizzle: the upper 64
    // columns of each 128 therefore use the other 8-byte half of every chunk (swapped
    // back on the way out), so that a quarter-wave covers all banks once.
    constexpr bool SUBSWZ = RPT * RB / 8 == 8;
    auto stage_off = [&](int j) {
      const int cl = lcol + j;
      const int half = SUBSWZ ? ((cl >> 6) & 1) << 3 : 0;
      return cl * BPC + ((((byte0 >> 4) ^ ((cl >> 3) & (CPC - 1))) << 4) | ((byte0 & 15) ^ half));
    };
    if constexpr (SR && !BF16) {
      // FP32 with stochastic rounding: 4 rows' draws at a time, all columns of them.
      // Lanes t and t ^ 1 share one Philox block per row only when cols % 8 == 0; a
      // column-only cast may have cols % 8 == 4, where every other row's blocks start
      // at odd lanes, and each lane then draws its own rows' blocks.
      const bool pairs = (Cu & 7u) == 0u;
      uint32_t w[VEC][RPT / 4];
#pragma unroll
      for (int g = 0; g < RPT / 4; ++g) {
        uint32_t dr[4][VEC / 2];
        if (pairs) {
          row_draws_pair(4 * g, dr[0], dr[1]);
          row_draws_pair(4 * g + 2, dr[2], dr[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) row_draws(4 * g + r, dr[r]);
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int e = int(code_j[j]) - 127;
          float f[4];
          uint32_t xb[4], uu[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xb[r] = (&v[4 * g + r].x)[j];
            uu[r] = (j & 1) ? (dr[r][j >> 1] >> 16) : (dr[r][j >> 1] & 0xFFFFu);
          }
          sr_scaled_n<F, 4, SRFAST>(xb, e, uu, f);
          w[j][g] = encode4_f32<F, M>(f[0], f[1], f[2], f[3], sr_enc_code(code_j[j]));
        }
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        if constexpr (RPT == 16 && RB == 8) {
          *reinterpret_cast<uint4*>(lds_codes + stage_off(j)) = make_uint4(w[j][0], w[j][1], w[j][2], w[j][3]);
        } else if constexpr (RPT == 16) {
          *reinterpret_cast<uint2*>(lds_codes + stage_off(j)) =
              make_uint2((w[j][0] & 0xFFFFu) | (w[j][1] << 16), (w[j][2] & 0xFFFFu) | (w[j][3] << 16));
        } else if constexpr (RB == 8) {                          // narrow tiles: 8 rows
          *reinterpret_cast<uint2*>(lds_codes + stage_off(j)) = make_uint2(w[j][0], w[j][1]);
        } else {
          *reinterpret_cast<uint32_t*>(lds_codes + stage_off(j)) = (w[j][0] & 0xFFFFu) | (w[j][1] << 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ((SR && !BF16) ? 0 : VEC); ++j) {
      const int off = stage_off(j);
      if constexpr (BF16) {
        const int d = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t pr[4];
#pragma unroll
        for (int k = 0; k < RPT; k += 2) pr[k / 2] = __builtin_amdgcn_perm((&v[k + 1].x)[d], (&v[k].x)[d], sel);
        uint2 w;
        if constexpr (SR) {
          // rows 0..7 of column j: the element draw is half (j & 1) of word j >> 1 of each row
          uint32_t dj[RPT];
#pragma unroll
          for (int k = 0; k < RPT; ++k) dj[k] = (j & 1) ? (draw[KEEP ? k : 0][j >> 1] >> 16) : (draw[KEEP ? k : 0][j >> 1] & 0xFFFFu);
          w = encode_col_sr<F, M, SRFAST>(pr, dj, code_j[j]);
        } else {
          w = encode8_bf16<F, M>(pr[0], pr[1], pr[2], pr[3], code_j[j]);
        }
        if constexpr (RB == 8) *reinterpret_cast<uint2*>(lds_codes + off) = w;       // 8 rows
        else *reinterpret_cast<uint32_t*>(lds_codes + off) = w.x;                   // 8 rows in 4 bytes
      } else {
        uint32_t w[RPT / 4];
#pragma unroll
        for (int g = 0; g < RPT / 4; ++g)
          w[g] = encode4_f32<F, M>(__uint_as_float((&v[4 * g].x)[j]), __uint_as_float((&v[4 * g + 1].x)[j]),
                                   __uint_as_float((&v[4 * g + 2].x)[j]), __uint_as_float((&v[4 * g + 3].x)[j]),
                                   code_j[j]);
        if constexpr (RPT == 16 && RB == 8) {
          *reinterpret_cast<uint4*>(lds_codes + off) = make_uint4(w[0], w[1], w[2], w[3]);   // 16 rows
        } else if constexpr (RPT == 16) {
          *reinterpret_cast<uint2*>(lds_codes + off) =
              make_uint2((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16));
        } else if constexpr (RB == 8) {                                                   // 8 rows
          *reinterpret_cast<uint2*>(lds_codes + off) = make_uint2(w[0], w[1]);
        } else {
          *reinterpret_cast<uint32_t*>(lds_codes + off) = (w[0] & 0xFFFFu) | (w[1] << 16);
        }
      }
    }
    if (q == 0) {
      if constexpr (VEC == 8) {
        *reinterpret_cast<uint2*>(lds_scales + wr * TC + lcol) =
            make_uint2(pack_low_bytes(code_j[0], code_j[1], code_j[2], code_j[3]),
                       pack_low_bytes(code_j[4], code_j[5], code_j[6], code_j[7]));
      } else {
        *reinterpret_cast<uint32_t*>(lds_scales + wr * TC + lcol) =
            pack_low_bytes(code_j[0], code_j[1], code_j[2], code_j[3]);
      }
    }
    __syncthreads();

    // transposed write-out: tile column cl -> row (c0 + cl) of the column plane;
    // 16 staged bytes (ROWS_PER_CHUNK rows) go out as 16 bytes, or 12 once packed to 6 bits
    constexpr int ROWS_PER_CHUNK = 16 * 8 / RB;
    constexpr uint32_t OUT_CHUNK = 16 * CB / RB;
    const uint32_t Ru = uint32_t(R);
    const uint32_t cpitch = Ru * CB / 8;              // column-plane row pitch in bytes (< 2^23)
    const int64_t ctile_elem = (int64_t(bi) * C + c0) * R + r0;
    uint8_t* cct = reinterpret_cast<uint8_t*>(a.col_codes) + ctile_elem * CB / 8;
    // Every staged chunk, this thread's column-scale dword and its row-scale word are read
    // from LDS before the first store (all these LDS addresses exist whatever the tile's
    // extent), so the reads overlap instead of each waiting behind the previous store.
    constexpr int NWO = TC * CPC / kThreads;
    uint4 wo[NWO];
#pragma unroll
    for (int i = 0; i < NWO; ++i) {
      const int id = threadIdx.x + i * kThreads;
      const int cl = id / CPC, part = id % CPC;
      const uint4 w = *reinterpret_cast<const uint4*>(lds_codes + cl * BPC + ((part ^ ((cl >> 3) & (CPC - 1))) << 4));
      // the chunk halves of the upper 64 columns of each 128 (SUBSWZ); with 512 threads and
      // 8 chunks per column, column cl = (threadIdx.x + 512 i) / 8 has (cl / 64) & 1 == i & 1
      const bool swap = SUBSWZ && ((CPC == 8 && kThreads == 512) ? (i & 1) != 0 : ((cl >> 6) & 1) != 0);
      wo[i] = swap ? make_uint4(w.z, w.w, w.x, w.y) : w;
    }
    // the column's 4 block codes (one per wave row), byte w for rows 32 w .. 32 w + 31
    auto col_codes4 = [&](int c) {
      return uint32_t(lds_scales[c]) | (uint32_t(lds_scales[TC + c]) << 8) | (uint32_t(lds_scales[2 * TC + c]) << 16) |
             (uint32_t(lds_scales[3 * TC + c]) << 24);
    };
    static_assert(kWaveRows == 4, "a column's block codes fill one dword");
    const uint32_t col_scale_dw = B2 ? 0u : col_codes4(int(threadIdx.x & (TC - 1)));
    uint2 row_scale_qw = make_uint2(0u, 0u);
    if constexpr (RS8) {
      const int rl = threadIdx.x & (kTileR - 1);
      row_scale_qw = make_uint2(lds_rs[2 * rl], lds_rs[2 * rl + 1]);
    }
    if constexpr (CB == 6) {
#pragma unroll
      for (int i = 0; i < NWO; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int cl = id / CPC;
        const int part = id % CPC;
        if (cl < cols_in && part * ROWS_PER_CHUNK < rows_in) {
          const uint3 p = pack6x16(wo[i].x, wo[i].y, wo[i].z, wo[i].w);
          store12(cct + uint32_t(cl) * cpitch + uint32_t(part) * OUT_CHUNK, p.x, p.y, p.z);
        }
      }
      if (rs8 && int(threadIdx.x) < rows_in) {
        // the staged row scales: one 8-byte word (256 columns) per tile row
        const int rl = threadIdx.x;
        store_sc1_8(a.row_scales + tile_elem / 32 + uint32_t(rl) * (Cu / 32), row_scale_qw.x, row_scale_qw.y);
      }
    } else {
      // A wave's store covers the 64 / CPC columns from its first one, cl0: the descriptor
      // starts there and spans 64 / CPC column pitches (below 2^27 bytes).
#pragma unroll
      for (int i = 0; i < NWO; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int cl = id / CPC;
        const int part = id % CPC;
        const int cl0 = __builtin_amdgcn_readfirstlane((int(threadIdx.x & ~63u) + i * kThreads) / CPC);
        const __amdgpu_buffer_rsrc_t r = plane_rsrc(cct + uint32_t(cl0) * cpitch, uint32_t(64 / CPC) * cpitch);
        const bool ok = cl < cols_in && part * ROWS_PER_CHUNK < rows_in;
        bstore_nt16(r, ok ? uint32_t(cl - cl0) * cpitch + uint32_t(part) * OUT_CHUNK : kOutOfRange, wo[i]);
      }
      if (rs8) {
        // the staged row scales: one 8-byte word (256 columns) per tile row; the tile's
        // 128 rows of the row-scale plane (cols % 256 == 0 here)
        const __amdgpu_buffer_rsrc_t r = plane_rsrc(a.row_scales + tile_elem / 32, uint32_t(kTileR) * (Cu / 32));
        bstore8(r, int(threadIdx.x) < rows_in ? uint32_t(threadIdx.x) * (Cu / 32) : kOutOfRange, row_scale_qw);
      }
    }
    if (lines6) {
      // the staged 6-bit row codes: 12 chunks of 16 bytes per tile row, through L2
      // (lines at the tile's edges are shared with the neighbouring tile). With
      // cols % 64 == 0 a ragged tile holds 48, 96 or 144 bytes per row, whole
      // chunks; the 8-byte branch only guards a partial one.
      uint8_t* rct = reinterpret_cast<uint8_t*>(a.row_codes) + tile_elem * 6 / 8;
      const uint32_t rpitch = Cu * 6 / 8;
      const int bytes_in = cols_in * 6 / 8;
#pragma unroll
      for (int i = 0; i < kTileR * 12 / kThreads; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int rl = id / 12, part = id % 12;
        if (rl < rows_in && 16 * part < bytes_in) {
          const uint4 w = *reinterpret_cast<const uint4*>(lds_rows6 + rl * P6 + 16 * part);
          uint8_t* dst = rct + uint32_t(rl) * rpitch + uint32_t(16 * part);
          if (16 * part + 16 <= bytes_in) *reinterpret_cast<uint4*>(dst) = w;
          else *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);
        }
      }
    }
    if constexpr (ROWLDS) {
      // the staged row codes: 8 lanes write one tile row's 128 bytes (256 columns)
      uint8_t* rct = reinterpret_cast<uint8_t*>(a.row_codes) + tile_elem / 2;
      const __amdgpu_buffer_rsrc_t r = plane_rsrc(rct, uint32_t(kTileR) * (Cu / 2));
#pragma unroll
      for (int i = 0; i < kTileR * 8 / kThreads; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int rl = id >> 3, part = id & 7;
        const uint4 w = *reinterpret_cast<const uint4*>(lds_rows + rl * (kTileC / 2) + ((part ^ ((rl >> 3) & 7)) << 4));
        const bool ok = rl < rows_in && 32 * part < cols_in;
        bstore_nt16(r, ok ? uint32_t(rl) * (Cu / 2) + uint32_t(16 * part) : kOutOfRange, w);
      }
    }
    if constexpr (B2) {
      // 32x32 blocks: column block cb of the tile, row blocks r0/32 .. +3 of the [C/32][R/32] grid
      const int cb = threadIdx.x;
      if (cb < kTileC / 32 && 32 * cb < cols_in) {
        const int64_t nbr = R / 32;
        uint8_t* dst = a.col_scales + (int64_t(bi) * (C / 32) + c0 / 32 + cb) * nbr + r0 / 32;
        if (a.flags & kColScaleDword) {
          *reinterpret_cast<uint32_t*>(dst) = col_codes4(32 * cb);
        } else {
#pragma unroll
          for (int w = 0; w < kWaveRows; ++w)
            if (32 * w < rows_in) dst[w] = lds_scales[w * TC + 32 * cb];
        }
      }
    } else if (a.flags & kColScaleDword) {
      // the tile's columns of the column-scale plane (rows % 128 == 0 here)
      const __amdgpu_buffer_rsrc_t r = plane_rsrc(a.col_scales + ctile_elem / 32, uint32_t(TC) * (Ru / 32));
      const int cl = threadIdx.x;
      bstore4(r, cl < cols_in ? uint32_t(cl) * (Ru / 32) : kOutOfRange, col_scale_dw);
    } else if (int(threadIdx.x) < cols_in) {
      const int cl = threadIdx.x;
      uint8_t* dst = a.col_scales + ctile_elem / 32 + uint32_t(cl) * Ru / 32;
#pragma unroll
      for (int w = 0; w < kWaveRows; ++w)
        if (32 * w < rows_in) dst[w] = lds_scales[w * TC + cl];
    }
  }
}

// Row-wise only: the blocks are 32 consecutive elements of the flat
// [batch][rows][cols] order, so the cast is a linear stream. Lane i of a wave
// handles 16-byte chunk i of each 1 KiB wave step (4 (BF16) or 8 (FP32) lanes
// per block); kRowSteps steps per wave are in flight at once. The 4 scale
// bytes of 4 neighbouring blocks are ORed into one dword store.

template <bool BF16, int F, int M, int RD>
__global__ __launch_bounds__(kRowThreads) void mx_cast_rows_kernel(CastArgs a, int64_t nchunks) {
  constexpr int VEC = InC<BF16>::vec;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int LPB = 32 / VEC;                 // lanes per block: 4 | 8
  constexpr int LPG = 4 * LPB;                  // lanes per 4-block scale group: 16 | 32
  constexpr int CB = FmtC<F>::bits;
  const int lane = threadIdx.x & 63;
  const int64_t wave_global = int64_t(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  const int64_t chunk0 = wave_global * (64 * kRowSteps) + lane;
  const uint8_t* x = reinterpret_cast<const uint8_t*>(a.x);
  uint8_t* rc = reinterpret_cast<uint8_t*>(a.row_codes);

  uint4 v[kRowSteps];
#pragma unroll
  for (int u = 0; u < kRowSteps; ++u) {
    const int64_t ch = chunk0 + 64 * u;
    const bool ok = ch < nchunks;
    const uint4 d = load_nt(x + (ok ? ch : 0) * 16);
    v[u] = ok ? d : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < kRowSteps; ++u) {
    const int64_t ch = chunk0 + 64 * u;
    uint32_t m;
    if constexpr (BF16) {
      const uint32_t h = pk_max_u16(pk_max_u16(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                    pk_max_u16(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu));
      m = max(h & 0xFFFFu, h >> 16);
    } else {
      m = max(max(v[u].x & 0x7FFFFFFFu, v[u].y & 0x7FFFFFFFu), max(v[u].z & 0x7FFFFFFFu, v[u].w & 0x7FFFFFFFu));
    }
    m = group_max<LPB>(m);
    const uint32_t code = scale_code<F, M, BF16>(m);
    const int64_t e0 = ch * VEC;                       // first element of this chunk
    uint8_t* dst = rc + e0 * CB / 8;
    uint32_t draw[RD == kSr ? VEC / 2 : 1];
    if constexpr (RD == kSr) {
      const uint4 w = sr_words(uint64_t(e0) >> 3, a.seed_lo, a.seed_hi);
      const int h = int(e0 & 7) >> 1;
#pragma unroll
      for (int j = 0; j < VEC / 2; ++j) draw[j] = (h + j) == 0 ? w.x : (h + j) == 1 ? w.y : (h + j) == 2 ? w.z : w.w;
    }
    if constexpr (BF16) {
      const uint2 w = RD == kSr ? encode8_sr<true, F, M, true>(v[u], draw, code) : encode8_bf16<F, M>(v[u].x, v[u].y, v[u].z, v[u].w, code);
      if constexpr (CB == 6) {
        // even lanes store their 48 bits and the odd neighbour's as 12 bytes
        const uint32_t hi = pack6(w.y);
        const uint32_t p0 = pack6(w.x) | (hi << 24), p1 = hi >> 8;
        const uint32_t o0 = dpp<kDppXor1>(p0), o1 = dpp<kDppXor1>(p1);
        if (ch < nchunks && (lane & 1) == 0) store_nt12(dst, p0, p1 | (o0 << 16), (o0 >> 16) | (o1 << 16));
      } else if (ch < nchunks) {
        if constexpr (CB == 8) store_nt8(dst, w);
        else store_nt4(dst, w.x);
      }
    } else {
      const uint32_t w = RD == kSr ? encode8_sr<false, F, M, true>(v[u], draw, code).x
                                   : encode4_f32<F, M>(__uint_as_float(v[u].x), __uint_as_float(v[u].y),
                                                       __uint_as_float(v[u].z), __uint_as_float(v[u].w), code);
      if constexpr (CB == 6) {
        // lane 4i stores the 24 bits of lanes 4i .. 4i+3 as 12 bytes
        const uint32_t g0 = pack6(w);
        const uint32_t g1 = dpp<kDppQuadNext>(g0), g2 = dpp<kDppXor2>(g0), g3 = dpp<kDppQuadPrev>(g0);
        if (ch < nchunks && (lane & 3) == 0)
          store_nt12(dst, g0 | (g1 << 24), (g1 >> 8) | (g2 << 16), (g2 >> 16) | (g3 << 8));
      } else if (ch < nchunks) {
        if constexpr (CB == 8) store_nt4(dst, w);
        else store_nt2(dst, w);
      }
    }
    // scale bytes of the 4 blocks of this lane's group, lane 0 of the group stores
    uint32_t sb = code << (8 * ((lane % LPG) / LPB));
    if constexpr (BF16) {
      sb |= dpp<kDppRor4>(sb);
      sb |= dpp<kDppRor8>(sb);
    } else {
      sb |= dpp<kDppRor8>(sb);
      sb = or_xor16(sb);
    }
    if ((lane % LPG) == 0 && ch < nchunks) {
      const int64_t blk = e0 / 32;                     // multiple of 4
      const int64_t nblk = nchunks / LPB;
      if ((a.flags & kRowScaleDword) && blk + 4 <= nblk) {
        *reinterpret_cast<uint32_t*>(a.row_scales + blk) = sb;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (blk + b < nblk) a.row_scales[blk + b] = uint8_t(sb >> (8 * b));
      }
    }
  }
}

template <bool BF16, int F, int M, int RD>
hipError_t launch_rows(const CastArgs& a, int64_t nchunks, hipStream_t s) {
  const int64_t per_block = int64_t(kRowThreads / 64) * 64 * kRowSteps;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  return launch_kernel(mx_cast_rows_kernel<BF16, F, M, RD>, dim3(uint32_t(blocks)), dim3(kRowThreads), s, a,
                       nchunks);
}

template <bool BF16, int F, int M, int AX, int RD, bool B2>
hipError_t launch_one(const CastArgs& a, uint32_t nblocks, hipStream_t s) {
  return launch_kernel(mx_cast_kernel<BF16, F, M, AX, RD, B2>, dim3(nblocks), dim3(kThreads), s, a);
}

// Row-only casts with 1x32 blocks are a linear stream (mx_cast_rows_kernel);
// everything else runs the tiled kernel.
template <bool BF16, int F, int M, int RD, bool B2>
hipError_t by_axis(int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  switch (axis) {
    case kRow:
      if constexpr (B2) return launch_one<BF16, F, M, kRow, RD, true>(a, nb, s);
      else return launch_rows<BF16, F, M, RD>(a, a.elements / InC<BF16>::vec, s);
    case kCol: return launch_one<BF16, F, M, kCol, RD, B2>(a, nb, s);
    default: return launch_one<BF16, F, M, kBoth, RD, B2>(a, nb, s);
  }
}

template <bool BF16, int F, int RD, bool B2>
hipError_t by_mode(int mode, int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  return mode == kRoundUp ? by_axis<BF16, F, kRoundUp, RD, B2>(axis, a, nb, s)
                          : by_axis<BF16, F, kFloor, RD, B2>(axis, a, nb, s);
}

template <bool BF16, int RD, bool B2>
hipError_t by_fmt(int fmt, int mode, int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  switch (fmt) {
    case kE4M3: return by_mode<BF16, kE4M3, RD, B2>(mode, axis, a, nb, s);
    case kE5M2: return by_mode<BF16, kE5M2, RD, B2>(mode, axis, a, nb, s);
    case kE2M1: return by_mode<BF16, kE2M1, RD, B2>(mode, axis, a, nb, s);
    case kE2M3: return by_mode<BF16, kE2M3, RD, B2>(mode, axis, a, nb, s);
    case kE3M2: return by_mode<BF16, kE3M2, RD, B2>(mode, axis, a, nb, s);
    case kInt8: return by_mode<BF16, kInt8, RD, B2>(mode, axis, a, nb, s);
    default: return hipErrorInvalidValue;
  }
}

template <int RD, bool B2>
hipError_t launch_variant(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a, uint32_t nblocks,
                          hipStream_t s) {
  return in_bf16 ? by_fmt<true, RD, B2>(fmt, mode, axis, a, nblocks, s)
                 : by_fmt<false, RD, B2>(fmt, mode, axis, a, nblocks, s);
}

}  // namespace
}  // namespace mx
