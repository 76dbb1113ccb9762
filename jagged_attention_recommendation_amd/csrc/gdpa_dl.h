// Direct-load tiles for D = 128 bf16: 64 rows x 256 bytes in LDS, filled by
// buffer_load_dwordx4 ... lds (each lane's 16 bytes go straight to LDS at base + 16 * lane: no
// staging registers, no LDS store instructions).
//
// Rows have no padding; the 16-byte chunk c of row r sits at chunk c ^ f(r),
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3). One direct-load instruction fills four consecutive
// rows, and each lane fetches the global chunk that belongs at its slot. Row reads (16 rows, one
// chunk each) and transposed reads (4 rows x 4 chunks per half-wave) then hit 16 distinct
// 16-byte bank groups. Rows past the end of a sample are fetched from its first row: finite
// values that the kernels mask, so no tile needs zero filling.
#pragma once

#include "gdpa_common.h"

namespace gdpa {
namespace dl {

constexpr int D = 128;
constexpr int ROWS = 64;
constexpr int ROWB = 256;            // bytes per tile row
constexpr int TILE = ROWS * ROWB;    // 16 KiB

__device__ __forceinline__ int xf(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int xoff(int r, int chunk) { return r * ROWB + ((chunk ^ xf(r)) << 4); }

// MFMA operand whose k runs along D: lane reads row rbase + l%32, k-step s (chunk 2s + l/32).
__device__ __forceinline__ bf16x8 row_op(const GDPA_LDS char* t, int rbase, int s, int lane) {
  return *(const GDPA_LDS bf16x8*)(t + xoff(rbase + (lane & 31), 2 * s + (lane >> 5)));
}

// MFMA operand whose k runs along the rows (ds_read_b64_tr_b16): D index n*32 + l%32, rows
// row0 + 4g + {0..3} and row0 + 8 + 4g + {0..3} (g = l/32), the k order of registers
// 8*s2..8*s2+7 of a 32x32 accumulator block when row0 = 16*s2 within the block.
__device__ __forceinline__ bf16x8 tr_op(const GDPA_LDS char* t, int row0, int n, int lane) {
  const int i16 = lane & 15, q = i16 & 3;
  const int rr = row0 + 4 * (lane >> 5) + (i16 >> 2);
  const int c = 4 * n + 2 * ((lane >> 4) & 1) + (q >> 1);
  const int within = 8 * (q & 1);
  const i16x4 lo = lds_read_tr(t + xoff(rr, c) + within);
  const i16x4 hi = lds_read_tr(t + xoff(rr + 8, c) + within);
  return cat_tr(lo, hi);
}

// Issue the direct loads of rows r0 .. r0 + 63 of head h of a jagged [rows, H, 128] tensor whose
// sample starts at row base and has L > r0 rows, into an LDS tile. Workgroups of 4 waves:
// thread (wave w, lane l) fills, for u = 0..3, physical row 16u + 4w + l/16 at chunk l%16.
// The loads are buffer loads through a resource that starts at row r0 and ends with the tile's
// last valid row (every offset stays below 64 x H x 256 bytes); rows at or past L are fetched
// from row r0. The buffer form, unlike the global form, leaves the LDS-read wait counts exact.
__device__ __forceinline__ void issue_tile(GDPA_LDS char* __restrict__ stage, const __bf16* src, int r0,
                                           int L, int base, int H, int h, int w, int lane) {
  const __bf16* p = src + ((int64_t)(base + r0) * H + h) * D;
  const int n = min(ROWS, L - r0);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, ((n - 1) * H + 1) * ROWB, 0x00020000);
  const int rsub = 4 * w + (lane >> 4);
  const int c = (lane & 15) ^ xf(rsub);  // xf depends on the row only through r mod 16
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int row = 16 * u + rsub;
    row = row < n ? row : 0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GDPA_LDS void*)(stage + (16 * u + 4 * w) * ROWB), 16,
                                             row * H * ROWB + c * 16, 0, 0, 0);
  }
}

// Issues the direct loads that fill win[t] = table[clamp(d0 + dir * t, 0, n - 1)] for t in
// [0, cnt), raw (the caller scales them after its wait), rounded up to whole waves of 64
// entries: wave w, lane l fills entry 256 k + 64 w + l with its k-th load. The window buffer
// must hold cnt rounded up to a multiple of 64.
__device__ __forceinline__ void issue_window(GDPA_LDS float* win, const float* table, int n, int d0, int dir,
                                             int cnt, int w, int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)table, (short)0, n * 4, 0x00020000);
  for (int k = 0; 256 * k + 64 * w < cnt; ++k) {
    const int d = clampi(d0 + dir * (256 * k + 64 * w + lane), 0, n - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GDPA_LDS void*)(win + 256 * k + 64 * w), 4, d * 4, 0, 0, 0);
  }
}

}  // namespace dl
}  // namespace gdpa
