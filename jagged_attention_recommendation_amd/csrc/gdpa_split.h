// Fixed-order combines of split tiles (bf16 paths).
//
// When a few long tiles would leave most compute units idle, the scheduler splits each of them
// into chunks of inner tiles (page "GEM Training: How Meta Doubled the Efficiency of Its
// LLM-Scale Ads Foundation Model", JFA and GDPA paragraphs: short sequences must not idle the
// GPU, and the scheduling was redesigned for large batches and asymmetric lengths). Each chunk
// writes fp32 partial rows to its slot and then counts itself done on the tile's counter; the
// workgroup that completes the count combines the tile's chunks in chunk order, so results do
// not depend on which chunk finished last:
//   softmax forward: with per-chunk running max m_c (log2 units), sum l_c and unnormalised O_c,
//     m = max_c m_c, w_c = 2^(m_c - m), l = sum_c w_c l_c, O = sum_c w_c O_c / l,
//     lse = (m + log2 l) ln 2  (the online-softmax rescaling, applied across chunks);
//   GDPA forward: O = sum_c O_c;
//   dQ = scale * sum_c dQ_c;  dK = scale * sum_c dK_c;  dV = sum_c dV_c.
// Thread pair (2r, 2r + 1) of the 256-thread workgroup owns tile row r, D / 2 columns each.
#pragma once

#include <math.h>

#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {
namespace split {

constexpr int ROWS = 128;  // rows per tile in every split list
static_assert(FWD_BM_BF16 == ROWS && BWD_Q_ITEM == ROWS && BWD_K_ITEM == ROWS, "tile rows");

// Item::chunk holds the chunk index in its low 16 bits and the tile's chunk count above them.
__device__ __forceinline__ int chunk_index(int packed) { return packed & 0xffff; }
__device__ __forceinline__ int chunk_count(int packed) { return packed >> 16; }

// Called by every thread of the workgroup after its partial rows are written: returns true in
// the workgroup that completes the tile (all its chunks' partials are then visible to it).
__device__ __forceinline__ bool chunk_done(int* counter, int n, GDPA_LDS int* flag_lds) {
  __threadfence();  // this thread's partial rows reach the device-coherent level
  __syncthreads();
  if (threadIdx.x == 0) *flag_lds = atomicAdd(counter, 1) == n - 1;
  __syncthreads();
  const bool last = *flag_lds != 0;
  if (last) __threadfence();  // and the other chunks' rows are seen
  return last;
}

// acc[0..N) += w * src[0..N) (16-byte loads)
template <int N>
__device__ __forceinline__ void axpy(float* acc, float w, const float* src) {
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const f32x4 v = *(const f32x4*)(src + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[4 * j + e] = fmaf(w, v[e], acc[4 * j + e]);
  }
}

// dst[0..N) = bf16(acc * mul)
template <int N>
__device__ __forceinline__ void store(__bf16* dst, const float* acc, float mul) {
#pragma unroll
  for (int j = 0; j < N / 8; ++j) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = acc[8 * j + e] * mul;
    *(bf16x8*)(dst + 8 * j) = pack8(t);
  }
}

template <bool SOFTMAX, int D = 128>
__device__ void combine_fwd_tile(const FwdArgs& a, int b, int tile, int h, int n, int slot) {
  constexpr int N = D / 2;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int r = threadIdx.x >> 1, c0 = (threadIdx.x & 1) * N;
  const int iq = tile * ROWS + r;
  if (iq >= Lq) return;
  float m = -INFINITY, l = 0.0f;
  if (SOFTMAX)
    for (int k = 0; k < n; ++k) m = fmaxf(m, a.part_ml[(int64_t)(slot + k) * 2 * ROWS + r]);
  float acc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) acc[j] = 0.0f;
  for (int k = 0; k < n; ++k) {
    float wk = 1.0f;
    if (SOFTMAX) {
      const float mk = a.part_ml[(int64_t)(slot + k) * 2 * ROWS + r];
      wk = mk == -INFINITY ? 0.0f : fast_exp2(mk - m);
      l = fmaf(wk, a.part_ml[(int64_t)(slot + k) * 2 * ROWS + ROWS + r], l);
    }
    axpy<N>(acc, wk, a.part_o + ((int64_t)(slot + k) * ROWS + r) * D + c0);
  }
  const int64_t orow = (int64_t)(q0 + iq) * a.H + h;
  store<N>((__bf16*)a.O + orow * D + c0, acc, SOFTMAX ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f);
  if (SOFTMAX && c0 == 0 && a.lse != nullptr) a.lse[orow] = l > 0.0f ? (m + log2f(l)) * LN2 : -INFINITY;
}

template <int D = 128>
__device__ inline void combine_dq_tile(const BwdArgs& a, int b, int tile, int h, int n, int slot) {
  constexpr int N = D / 2;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int r = threadIdx.x >> 1, c0 = (threadIdx.x & 1) * N;
  const int iq = tile * ROWS + r;
  if (iq >= Lq) return;
  float acc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) acc[j] = 0.0f;
  for (int k = 0; k < n; ++k) axpy<N>(acc, 1.0f, a.part_dq + ((int64_t)(slot + k) * ROWS + r) * D + c0);
  const int64_t row = (int64_t)(q0 + iq) * a.H + h;
  if (a.dq_f32) {  // shared Q: this sample's gradient, summed over samples afterwards
#pragma unroll
    for (int j = 0; j < N; j += 4)
      *(f32x4*)(a.dq_f32 + row * D + c0 + j) =
          f32x4{acc[j] * a.scale, acc[j + 1] * a.scale, acc[j + 2] * a.scale, acc[j + 3] * a.scale};
    return;
  }
  store<N>((__bf16*)a.dQ + row * D + c0, acc, a.scale);
}

__device__ inline void combine_dkdv_tile(const BwdArgs& a, int b, int tile, int h, int n, int slot) {
  constexpr int D = 128;
  const int kv0 = a.kv_off[b], Lk = a.kv_off[b + 1] - kv0;
  const int r = threadIdx.x >> 1, c0 = (threadIdx.x & 1) * 64;
  const int jk = tile * ROWS + r;
  if (jk >= Lk) return;
  const int64_t krow = ((int64_t)(kv0 + jk) * a.H + h) * D + c0;
  float acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.0f;
  for (int k = 0; k < n; ++k) axpy<64>(acc, 1.0f, a.part_dk + ((int64_t)(slot + k) * ROWS + r) * D + c0);
  store<64>((__bf16*)a.dK + krow, acc, a.scale);
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.0f;
  for (int k = 0; k < n; ++k) axpy<64>(acc, 1.0f, a.part_dv + ((int64_t)(slot + k) * ROWS + r) * D + c0);
  store<64>((__bf16*)a.dV + krow, acc, 1.0f);
}

}  // namespace split
}  // namespace gdpa
