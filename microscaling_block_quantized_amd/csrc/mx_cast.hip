// MX block quantization kernels: row-wise, column-wise and fused row+column.
//
// What is computed ("MXFP4 と NVFP4 は何が違うのか調べてみた" §2 and §4): every block
// of 32 elements gets one E8M0 scale 2^e chosen from the block's largest
// magnitude (OCP floor rule or the round-up rule), and each element is stored
// as x / 2^e in the element format with round-to-nearest-even and clipping at
// the format's largest value. Row blocks run along the contiguous axis;
// column blocks are 32 rows of one column and are written transposed, so the
// column copy is the row-wise quantization of X^T.
//
// One workgroup (4 waves) owns a 128-row x 128-column tile of one batch
// slice and reads it from HBM exactly once:
//   * lane = q * LPR + t: t picks a 16-byte column chunk (8 BF16 / 4 FP32),
//     q a group of RPT consecutive rows; wave w owns rows 32w .. 32w+31, so
//     one wave holds exactly one 32-row column block of the tile.
//   * row blocks: lane-local max, then a max over the 4 (BF16) or 8 (FP32)
//     lanes that share the block; codes go straight to HBM, 128 contiguous
//     bytes per row.
//   * column blocks: in-lane max over the thread's RPT rows, then a max over
//     the RG lanes that hold the other rows of the same 32-row block. The
//     1-byte codes (not the inputs) are staged in LDS as [column][row] so the
//     transposed plane is written in full 128-byte runs.
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kTileR = 128;
constexpr int kTileC = 128;
constexpr int kThreads = 256;
constexpr int kPitch = 144;      // LDS bytes per staged column (128 codes + pad)

// Hardware places workgroup i on XCD i % 8. Renumber so that each XCD walks a
// contiguous range of tiles; neighbouring tiles then share an L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nb) {
  const uint32_t xcd = bid & 7u, idx = bid >> 3;
  const uint32_t per = nb >> 3, rem = nb & 7u;
  return xcd * per + min(xcd, rem) + idx;
}

template <bool BF16, int F, int M, int AX>
__global__ __launch_bounds__(kThreads) void mx_cast_kernel(CastArgs a) {
  constexpr int VEC = InC<BF16>::vec;          // elements per 16-byte chunk
  constexpr int LPR = kTileC / VEC;            // lanes per tile row: 16 | 32
  constexpr int RG = 64 / LPR;                 // row groups per wave: 4 | 2
  constexpr int RPT = 32 / RG;                 // rows per thread: 8 | 16
  constexpr int LPB = 32 / VEC;                // lanes per row block: 4 | 8
  constexpr int CB = FmtC<F>::bits;            // code bits
  constexpr bool ROWS = (AX & kRow) != 0;
  constexpr bool COLS = (AX & kCol) != 0;

  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[COLS ? kTileC * kPitch : 16];
  __shared__ uint8_t lds_scales[COLS ? kTileC * 4 : 4];

  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t per_batch = a.tiles_r * a.tiles_c;
  const uint32_t bi = tile / per_batch;
  const uint32_t rem = tile - bi * per_batch;
  const uint32_t tr = rem / a.tiles_c;
  const int64_t r0 = int64_t(tr) * kTileR;
  const int64_t c0 = int64_t(rem - tr * a.tiles_c) * kTileC;
  const int64_t R = a.rows, C = a.cols;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int q = lane / LPR;
  const int t = lane % LPR;
  const int64_t col = c0 + int64_t(t) * VEC;
  const int64_t row_base = r0 + 32 * wave + RPT * q;
  const bool col_ok = col < C;

  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x) + (int64_t(bi) * R * C) * (BF16 ? 2 : 4);
  uint4 v[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int64_t row = row_base + k;
    if (col_ok && row < R)
      v[k] = *reinterpret_cast<const uint4*>(xb + (row * C + col) * (BF16 ? 2 : 4));
    else
      v[k] = make_uint4(0u, 0u, 0u, 0u);
  }

  // ---------------- row-wise blocks ----------------
  if constexpr (ROWS) {
    uint8_t* rc = reinterpret_cast<uint8_t*>(a.row_codes);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int64_t row = row_base + k;
      uint32_t m;
      if constexpr (BF16) {
        uint32_t h = pk_max_u16(pk_max_u16(v[k].x & 0x7FFF7FFFu, v[k].y & 0x7FFF7FFFu),
                                pk_max_u16(v[k].z & 0x7FFF7FFFu, v[k].w & 0x7FFF7FFFu));
        m = max(h & 0xFFFFu, h >> 16);
      } else {
        m = max(max(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu),
                max(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu));
      }
#pragma unroll
      for (int s = 1; s < LPB; s <<= 1) m = xor_max(m, s);
      const uint32_t code = scale_code<F, M, BF16>(m);
      const bool ok = col_ok && row < R;
      const int64_t e0 = (int64_t(bi) * R + row) * C + col;   // element index
      if constexpr (BF16) {
        const uint2 w = encode8_bf16<F, M>(v[k].x, v[k].y, v[k].z, v[k].w, code);
        if (ok) {
          if constexpr (CB == 8) *reinterpret_cast<uint2*>(rc + e0) = w;
          else *reinterpret_cast<uint32_t*>(rc + e0 / 2) = w.x;
        }
      } else {
        const uint32_t w = encode4_f32<F, M>(__uint_as_float(v[k].x), __uint_as_float(v[k].y),
                                             __uint_as_float(v[k].z), __uint_as_float(v[k].w), code);
        if (ok) {
          if constexpr (CB == 8) *reinterpret_cast<uint32_t*>(rc + e0) = w;
          else *reinterpret_cast<uint16_t*>(rc + e0 / 2) = uint16_t(w);
        }
      }
      if (ok && (t % LPB) == 0) a.row_scales[e0 / 32] = uint8_t(code);
    }
  }

  // ---------------- column-wise blocks ----------------
  if constexpr (COLS) {
    constexpr int CPL = CB == 8 ? RPT : RPT / 2;      // code bytes per column per thread
    const int row_in_tile = 32 * wave + RPT * q;        // first tile row of this thread
    uint32_t code_j[VEC];
    if constexpr (BF16) {
      uint32_t cm[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t* p0 = &v[0].x;
        cm[d] = p0[d] & 0x7FFF7FFFu;
      }
#pragma unroll
      for (int k = 1; k < RPT; ++k) {
        const uint32_t* pk = &v[k].x;
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], pk[d] & 0x7FFF7FFFu);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int s = LPR; s < 64; s <<= 1) cm[d] = xor_max_pk16(cm[d], s);
        code_j[2 * d] = scale_code<F, M, true>(cm[d] & 0xFFFFu);
        code_j[2 * d + 1] = scale_code<F, M, true>(cm[d] >> 16);
      }
      // encode: column j = 2d + h; rows k, k+1 paired via byte permute
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int d = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t pr[RPT / 2];
#pragma unroll
        for (int k = 0; k < RPT; k += 2) {
          const uint32_t* pa = &v[k].x;
          const uint32_t* pb = &v[k + 1].x;
          pr[k / 2] = __builtin_amdgcn_perm(pb[d], pa[d], sel);
        }
        const uint2 w = encode8_bf16<F, M>(pr[0], pr[1], pr[2], pr[3], code_j[j]);
        uint8_t* dst = lds_codes + (t * VEC + j) * kPitch + row_in_tile * CB / 8;
        if constexpr (CB == 8) *reinterpret_cast<uint2*>(dst) = w;
        else *reinterpret_cast<uint32_t*>(dst) = w.x;
      }
    } else {
      uint32_t cm[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t* p0 = &v[0].x;
        cm[d] = p0[d] & 0x7FFFFFFFu;
      }
#pragma unroll
      for (int k = 1; k < RPT; ++k) {
        const uint32_t* pk = &v[k].x;
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = max(cm[d], pk[d] & 0x7FFFFFFFu);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int s = LPR; s < 64; s <<= 1) cm[d] = xor_max(cm[d], s);
        code_j[d] = scale_code<F, M, false>(cm[d]);
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        uint32_t w[RPT / 4];
#pragma unroll
        for (int g = 0; g < RPT / 4; ++g) {
          const uint32_t* r0p = &v[4 * g].x;
          const uint32_t* r1p = &v[4 * g + 1].x;
          const uint32_t* r2p = &v[4 * g + 2].x;
          const uint32_t* r3p = &v[4 * g + 3].x;
          w[g] = encode4_f32<F, M>(__uint_as_float(r0p[j]), __uint_as_float(r1p[j]),
                                   __uint_as_float(r2p[j]), __uint_as_float(r3p[j]), code_j[j]);
        }
        uint8_t* dst = lds_codes + (t * VEC + j) * kPitch + row_in_tile * CB / 8;
        if constexpr (CB == 8) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          *reinterpret_cast<uint2*>(dst) =
              make_uint2((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16));
        }
      }
    }
    if (q == 0) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) lds_scales[(t * VEC + j) * 4 + wave] = uint8_t(code_j[j]);
    }
    __syncthreads();

    // transposed write-out: column c of the tile -> row (c0 + c) of the column plane
    constexpr int BPC = kTileR * CB / 8;               // code bytes per staged column
    constexpr int CPC = BPC / 16;                      // 16-byte chunks per column
    constexpr int ROWS_PER_CHUNK = 16 * 8 / CB;
    uint8_t* cc = reinterpret_cast<uint8_t*>(a.col_codes);
#pragma unroll
    for (int i = 0; i < kTileC * CPC / kThreads; ++i) {
      const int id = threadIdx.x + i * kThreads;
      const int cl = id / CPC;
      const int part = id % CPC;
      const int64_t oc = c0 + cl;
      const int64_t orow = r0 + int64_t(part) * ROWS_PER_CHUNK;
      if (oc < C && orow < R) {
        const uint4 w = *reinterpret_cast<const uint4*>(lds_codes + cl * kPitch + part * 16);
        const int64_t e0 = (int64_t(bi) * C + oc) * R + orow;
        *reinterpret_cast<uint4*>(cc + e0 * CB / 8) = w;
      }
    }
    if (threadIdx.x < kTileC) {
      const int cl = threadIdx.x;
      const int64_t oc = c0 + cl;
      if (oc < C) {
        uint8_t* dst = a.col_scales + ((int64_t(bi) * C + oc) * R + r0) / 32;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (r0 + 32 * w < R) dst[w] = lds_scales[cl * 4 + w];
      }
    }
  }
}

template <bool BF16, int F, int M, int AX>
hipError_t launch_one(const CastArgs& a, uint32_t nblocks, hipStream_t s) {
  hipLaunchKernelGGL((mx_cast_kernel<BF16, F, M, AX>), dim3(nblocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, int F, int M>
hipError_t by_axis(int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  switch (axis) {
    case kRow: return launch_one<BF16, F, M, kRow>(a, nb, s);
    case kCol: return launch_one<BF16, F, M, kCol>(a, nb, s);
    default: return launch_one<BF16, F, M, kBoth>(a, nb, s);
  }
}

template <bool BF16, int F>
hipError_t by_mode(int mode, int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  return mode == kRoundUp ? by_axis<BF16, F, kRoundUp>(axis, a, nb, s)
                          : by_axis<BF16, F, kFloor>(axis, a, nb, s);
}

template <bool BF16>
hipError_t by_fmt(int fmt, int mode, int axis, const CastArgs& a, uint32_t nb, hipStream_t s) {
  switch (fmt) {
    case kE4M3: return by_mode<BF16, kE4M3>(mode, axis, a, nb, s);
    case kE5M2: return by_mode<BF16, kE5M2>(mode, axis, a, nb, s);
    default: return by_mode<BF16, kE2M1>(mode, axis, a, nb, s);
  }
}

}  // namespace

CastGrid cast_grid(int64_t batch, int64_t rows, int64_t cols) {
  CastGrid g;
  g.tiles_r = (rows + kTileR - 1) / kTileR;
  g.tiles_c = (cols + kTileC - 1) / kTileC;
  g.blocks = batch * g.tiles_r * g.tiles_c;
  return g;
}

hipError_t launch_cast(bool in_bf16, int fmt, int mode, int axis, const CastArgs& a,
                       uint32_t nblocks, hipStream_t s) {
  return in_bf16 ? by_fmt<true>(fmt, mode, axis, a, nblocks, s)
                 : by_fmt<false>(fmt, mode, axis, a, nblocks, s);
}

}  // namespace mx
