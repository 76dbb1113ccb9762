// 64-row bf16 tiles in LDS, read two ways by the MFMA kernels:
//   * row reads: lane reads 16 bytes of logical row R (an A operand whose k runs along D);
//   * transposed reads (ds_read_b64_tr_b16): a 16-lane group reads 4 consecutive logical rows
//     x 32 bytes, and a half-wave 4 rows x 64 bytes (an A operand whose k runs along the rows).
// Row pitch is 2D + 16 bytes and logical row R sits at physical row
//   (R & ~15) | ((R & 3) << 2) | ((R >> 2) & 3)
// i.e. each 16-row block is stored with its 4x4 (row%4, row/4) grid transposed. Then the 16
// rows of a row read land on 16 distinct 16-byte bank groups, and the 4 rows of a transposed
// read on 4 distinct 64-byte bank groups (256-byte bank span).
#pragma once

#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

template <int D>
struct Tile {
  static constexpr int ROWS = 64;
  static constexpr int P = 2 * D + 16;
  static constexpr int BYTES = ROWS * P;
  static constexpr int CHUNKS = ROWS * D / 8;  // 16-byte chunks
  __device__ static __forceinline__ int prow(int r) {
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
  }
  // byte offset of (logical row r, element col)
  __device__ static __forceinline__ int off(int r, int col) { return prow(r) * P + col * 2; }
};

// A wave's 32 rows of one head of a jagged [rows, H, D] tensor (D = 32 or 64) in 32 x 2D bytes
// of LDS, filled by direct loads of 16 bytes per lane (whole rows, 64 / (D / 8) per instruction,
// no staging registers). Chunk c of row r sits at chunk c ^ sw(r), sw(r) = (r / (128 / 2D)) %
// (D / 8), so that an operand read (32 rows, one chunk each) spreads over all banks. Rows at or
// past the sample's end are fetched from the wave's first row: finite values the kernels mask.
template <int D>
struct WaveRows {
  static constexpr int RB = 2 * D;      // bytes per row
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per load instruction
  static constexpr int BYTES = 32 * RB;
  __device__ static __forceinline__ int sw(int r) { return (r / (128 / RB)) % CPR; }
  // rows r0 .. r0 + 31 (r0 < L) of the sample starting at row base
  __device__ static __forceinline__ void issue(GDPA_LDS char* dst, const __bf16* src, int r0, int L, int base,
                                               int H, int h, int lane) {
    const __bf16* p = src + ((int64_t)(base + r0) * H + h) * D;
    const int n = min(32, L - r0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, ((n - 1) * H + 1) * RB, 0x00020000);
#pragma unroll
    for (int u = 0; u < 32 / RPI; ++u) {
      const int r = RPI * u + lane / CPR;       // the row whose slot this lane fills
      const int c = (lane % CPR) ^ sw(r);       // the chunk that belongs in it
      const int rf = r < n ? r : 0;             // the row it is fetched from
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GDPA_LDS void*)(dst + RPI * u * RB), 16, rf * H * RB + c * 16,
                                               0, 0, 0);
    }
  }
  // MFMA operand whose k runs along D, k-step s: lane reads row l % 32, chunk 2s + l / 32
  __device__ static __forceinline__ bf16x8 op(const GDPA_LDS char* t, int s, int lane) {
    const int r = lane & 31, c = 2 * s + (lane >> 5);
    return *(const GDPA_LDS bf16x8*)(t + r * RB + ((c ^ sw(r)) << 4));
  }
};

// Global -> register staging of a 64-row tile of one head of a jagged tensor; rows at or beyond
// nrows (local) are zero. NT threads cooperate.
template <int D, int NT>
struct TileLoader {
  static constexpr int PER = Tile<D>::CHUNKS / NT;
  static_assert(PER >= 1 && Tile<D>::CHUNKS % NT == 0, "tile / thread count mismatch");
  i32x4 r[PER];
  __device__ __forceinline__ void load(const __bf16* src, int row0, int nrows, int base, int H,
                                       int h, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NT * u;
      const int row = c / (D / 8), col = c % (D / 8);
      if (row0 + row < nrows) {
        r[u] = *(const i32x4*)(src + ((int64_t)(base + row0 + row) * H + h) * D + col * 8);
      } else {
        r[u] = i32x4{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(GDPA_LDS char* dst, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NT * u;
      const int row = c / (D / 8), col = c % (D / 8);
      *(GDPA_LDS i32x4*)(dst + Tile<D>::off(row, col * 8)) = r[u];
    }
  }
};

// A operand (rows = tile rows rbase..rbase+31, k = D) for k-step s: lane reads logical row
// rbase + l%32, elements 16s + 8(l/32) .. +8.
template <int D>
__device__ __forceinline__ bf16x8 tile_row_op(const GDPA_LDS char* t, int rbase, int s, int lane) {
  return *(const GDPA_LDS bf16x8*)(t + Tile<D>::off(rbase + (lane & 31), 16 * s + 8 * (lane >> 5)));
}

// A operand of a transposed product (rows = D index n*32 + l%32, k = 8 tile rows): the 8 rows
// are key0 + 4(l/32) + {0..3} and key0 + 8 + 4(l/32) + {0..3}, matching the k order of an
// accumulator-derived B operand (registers 8*s2..8*s2+7 of a 32x32 block, key0 = 16*s2 within
// the block).
template <int D>
__device__ __forceinline__ bf16x8 tile_tr_op(const GDPA_LDS char* t, int key0, int n, int lane) {
  const int i16 = lane & 15;
  const int rr = key0 + 4 * (lane >> 5) + (i16 >> 2);
  const int col = n * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
  const i16x4 lo = lds_read_tr(t + Tile<D>::off(rr, col));
  const i16x4 hi = lds_read_tr(t + Tile<D>::off(rr + 8, col));
  return cat_tr(lo, hi);
}

// Store a lane's 32x32-block accumulator column (16 values, D index n*32 + (r/4)*8 + 4g + r%4)
// as bf16 into a row of a [rows, H, D] tensor, multiplied by mul.
__device__ __forceinline__ void store_acc_row_bf16(__bf16* row, const f32x16& acc, int n, int g,
                                                   float mul) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    bf16x2 lo = pack_bf16(acc[4 * r4 + 0] * mul, acc[4 * r4 + 1] * mul);
    bf16x2 hi = pack_bf16(acc[4 * r4 + 2] * mul, acc[4 * r4 + 3] * mul);
    bf16x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
    *(bf16x4*)(row + n * 32 + r4 * 8 + 4 * g) = v4;
  }
}

// Same as store_acc_row_bf16, in fp32.
__device__ __forceinline__ void store_acc_row_f32(float* row, const f32x16& acc, int n, int g,
                                                  float mul) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
    *(f32x4*)(row + n * 32 + r4 * 8 + 4 * g) =
        f32x4{acc[4 * r4] * mul, acc[4 * r4 + 1] * mul, acc[4 * r4 + 2] * mul, acc[4 * r4 + 3] * mul};
}

// Stage the bias of raw diagonals lo..hi (inclusive, unclamped: entry d holds
// bias[h][clamp(d, 0, nb - 1)]) in LDS, multiplied by mul, reversed (win[t] = entry hi - t) or in
// order (win[t] = entry lo + t), so lookups need no clamping. Returns false and stages nothing
// when the window is empty or wider than BIAS_WMAX (the caller then reads the table from global
// memory). The caller synchronises before reading.
__device__ __forceinline__ bool stage_bias_window(GDPA_LDS float* win, const float* bias_h, int nb,
                                                  int lo, int hi, bool reversed, float mul,
                                                  int tid, int nt) {
  const int n = hi - lo + 1;
  if (n <= 0 || n > BIAS_WMAX) return false;
  for (int t = tid; t < n; t += nt) win[t] = bias_h[clampi(reversed ? hi - t : lo + t, 0, nb - 1)] * mul;
  return true;
}

}  // namespace gdpa
