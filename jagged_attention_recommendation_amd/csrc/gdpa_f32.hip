// fp32 path: forward and backward with plain vector ALU arithmetic.
//
// Same definitions as the bf16 kernels (page "GEM Training: How Meta Doubled the Efficiency of
// Its LLM-Scale Ads Foundation Model": JFA and GDPA paragraphs), for fp32 tensors. This path is
// for small problems and exact-ish fp32 results: one thread per query (forward, dQ) or per key
// (dK/dV), keys / queries streamed through LDS in tiles of 64 rows. gfx950 has no fp32 matrix
// instruction faster than its vector units on these shapes, so no MFMA is used here.
// A causal sliding window (a.win = W > 0: key j is valid for query i when j > i - W) is one more
// mask term (the forward also starts at the first key tile the item's window reaches); a shared
// query block (a.q_shared) is read at row i for every sample, and the dQ kernel then writes each
// sample's fp32 gradient for the reduction over samples.
#include <math.h>

#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

namespace {

constexpr int TM = F32_BM;  // queries (or keys) per item, one per thread
constexpr int TN = F32_BN;  // rows per streamed tile

template <int D>
__device__ __forceinline__ void load_tile_f32(float (*dst)[D], const float* src, int row0, int nrows,
                                              int base, int H, int h, int tid) {
  // nrows valid rows starting at local row0; others zero-filled. float4 chunks.
  constexpr int CPR = D / 4;
  for (int c = tid; c < TN * CPR; c += 64) {
    int r = c / CPR, col = c % CPR;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row0 + r < nrows) v = *(const f32x4*)(src + ((int64_t)(base + row0 + r) * H + h) * D + col * 4);
    *(f32x4*)(&dst[r][col * 4]) = v;
  }
}

template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[TN][D];
  __shared__ __attribute__((aligned(16))) float Vs[TN][D];
  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items, 0, it)) return;
  const int h = it.h, H = a.H, tid = threadIdx.x;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int i = it.tile * TM + tid;
  const bool qv = i < Lq;
  const float* Q = (const float*)a.Q;
  const int64_t qin = a.q_shared ? (int64_t)i * H + h : (int64_t)(q0 + i) * H + h;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qv ? Q[qin * D + c] : 0.0f;
    o[c] = 0.0f;
  }
  int nkt = (Lk + TN - 1) / TN;
  if (CAUSAL) nkt = min(nkt, (min(Lq, (it.tile + 1) * TM) - 1) / TN + 1);
  const int win = a.win;
  float m = -INFINITY, l = 0.0f;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * a.nb : nullptr;
  for (int kt = win_first_ktile(it.tile * TM, win, TN); kt < nkt; ++kt) {
    __syncthreads();
    load_tile_f32<D>(Ks, (const float*)a.K, kt * TN, Lk, kv0, H, h, tid);
    load_tile_f32<D>(Vs, (const float*)a.V, kt * TN, Lk, kv0, H, h, tid);
    __syncthreads();
    for (int jj = 0; jj < TN; ++jj) {
      const int j = kt * TN + jj;
      if (j >= Lk || (CAUSAL && j > i) || (win > 0 && j <= i - win)) continue;
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) s += q[c] * Ks[jj][c];
      s *= a.scale;
      if (BIAS) s += bias_h[clampi(i - j, 0, a.nb - 1)];
      if (ACT == ACT_SOFTMAX) {
        const float m_new = fmaxf(m, s);
        const float corr = expf(m - m_new);
        const float pj = expf(s - m_new);
        l = l * corr + pj;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = o[c] * corr + pj * Vs[jj][c];
        m = m_new;
      } else {
        const float pj = act_fwd(ACT, s);
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] += pj * Vs[jj][c];
      }
    }
  }
  if (!qv) return;
  float inv = 1.0f;
  if (ACT == ACT_SOFTMAX) {
    inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (a.lse) a.lse[(int64_t)(q0 + i) * H + h] = l > 0.0f ? m + logf(l) : -INFINITY;
  }
  float* orow = (float*)a.O + ((int64_t)(q0 + i) * H + h) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4 v = {o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
    *(f32x4*)(orow + c) = v;
  }
}

// Gradient of one (query i, key j) score. Returns ds and writes p (the probability / activation).
template <int ACT>
__device__ __forceinline__ float score_grad(float s, float lse_i, float D_i, float dp, float& p) {
  if (ACT == ACT_SOFTMAX) {
    p = expf(s - lse_i);
    return p * (dp - D_i);
  }
  float y, dy;
  act_fwd_bwd(ACT, s, y, dy);
  p = y;
  return dp * dy;
}

// dQ (one thread per query) + the softmax row term D_i + per-item diagonal partials of dS for the
// bias gradient.
template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[TN][D];
  __shared__ __attribute__((aligned(16))) float Vs[TN][D];
  __shared__ float dS[TM][TN + 1];
  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items_q, 0, it)) return;
  const int h = it.h, H = a.H, tid = threadIdx.x;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int i0 = it.tile * TM;
  const int i = i0 + tid;
  const bool qv = i < Lq;
  const int64_t row = (int64_t)(q0 + (qv ? i : 0)) * H + h;
  const int64_t qin = a.q_shared ? (int64_t)(qv ? i : 0) * H + h : row;
  const int win = a.win;
  float q[D], dO[D], dq[D];
  float Di = 0.0f, lse_i = 0.0f;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qv ? ((const float*)a.Q)[qin * D + c] : 0.0f;
    dO[c] = qv ? ((const float*)a.dO)[row * D + c] : 0.0f;
    dq[c] = 0.0f;
  }
  if (ACT == ACT_SOFTMAX && qv) {
#pragma unroll
    for (int c = 0; c < D; ++c) Di += dO[c] * ((const float*)a.O)[row * D + c];
    lse_i = a.lse[row];
    a.Dvec[row] = Di;
  }
  int nkt = (Lk + TN - 1) / TN;
  if (CAUSAL) nkt = min(nkt, (min(Lq, i0 + TM) - 1) / TN + 1);
  // Bias gradient: the item's two 32-query row blocks own the partial rows
  // part[2 * tile + q, h, :] (tile = canonical query-tile index in it.aux). Diagonal c of a row
  // belongs to thread c % 64, which zeroes it here and later adds every contribution to it in a
  // fixed order. A row block's written range is the clamp of its raw diagonal range
  // [32rb - (k_end - 1), 32rb + 31], k_end = keys up to the last tile it can see.
  const int nb = a.nb;
  float* part[2] = {nullptr, nullptr};
  if (BIAS) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      part[q] = a.dbias_part + ((int64_t)h * a.part_rows + it.aux * 2 + q) * nb;
      const int wr = i0 + 32 * q;
      if (Lk > 0 && wr < Lq) {
        int last = nkt - 1;
        if (CAUSAL) last = min(last, (wr + 31) / TN);
        const int c_lo = clampi(wr - (last + 1) * TN + 1, 0, nb - 1);
        const int c_hi = clampi(wr + 31, 0, nb - 1);
        for (int c = c_lo + ((tid - c_lo % 64) + 64) % 64; c <= c_hi; c += 64) part[q][c] = 0.0f;
      }
    }
  }
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    load_tile_f32<D>(Ks, (const float*)a.K, kt * TN, Lk, kv0, H, h, tid);
    load_tile_f32<D>(Vs, (const float*)a.V, kt * TN, Lk, kv0, H, h, tid);
    __syncthreads();
    for (int jj = 0; jj < TN; ++jj) {
      const int j = kt * TN + jj;
      float ds = 0.0f;
      if (qv && j < Lk && !(CAUSAL && j > i) && !(win > 0 && j <= i - win)) {
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s += q[c] * Ks[jj][c];
          dp += dO[c] * Vs[jj][c];
        }
        s *= a.scale;
        if (BIAS) s += a.bias[(int64_t)h * nb + clampi(i - j, 0, nb - 1)];
        float p;
        ds = score_grad<ACT>(s, lse_i, Di, dp, p);
#pragma unroll
        for (int c = 0; c < D; ++c) dq[c] += ds * Ks[jj][c];
      }
      if (BIAS) dS[tid][jj] = ds;
    }
    if (BIAS) {
      __syncthreads();
      // Owner thread of clamped diagonal c is c % 64; per row block it sums, in a fixed order,
      // every raw diagonal rr = i - j of its 32 x 64 part of the tile that clamps to c.
      const int j0 = kt * TN;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int wr = i0 + 32 * q;
        if (wr >= Lq) continue;
        if (CAUSAL && j0 > wr + 31) continue;
        const int rr_lo = wr - (j0 + TN - 1), rr_hi = wr + 31 - j0;
        const int c_lo = clampi(rr_lo, 0, nb - 1), c_hi = clampi(rr_hi, 0, nb - 1);
        for (int c = c_lo + ((tid - c_lo % 64) + 64) % 64; c <= c_hi; c += 64) {
          const int a_lo = c == 0 ? rr_lo : c;  // raw diagonals mapping to c
          const int a_hi = c == nb - 1 ? rr_hi : c;
          float acc = 0.0f;
          for (int rr = max(a_lo, rr_lo); rr <= min(a_hi, rr_hi); ++rr) {
            // elements (ii, jj), ii in this row block, with (i0 + ii) - (j0 + jj) = rr
            const int d0 = rr - (i0 - j0);  // ii - jj
            const int ii_lo = max(32 * q, d0), ii_hi = min(32 * q + 31, TN - 1 + d0);
            for (int ii = ii_lo; ii <= ii_hi; ++ii) acc += dS[ii][ii - d0];
          }
          part[q][c] += acc;
        }
      }
    }
  }
  if (!qv) return;
  // a shared query block: this sample's gradient at O's row, summed over samples afterwards
  float* dqrow = (a.dq_f32 ? a.dq_f32 : (float*)a.dQ) + row * D;
#pragma unroll
  for (int c = 0; c < D; ++c) dqrow[c] = dq[c] * a.scale;
}

// dK, dV (one thread per key).
template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float Qs[TM][D];
  __shared__ __attribute__((aligned(16))) float dOs[TM][D];
  __shared__ float lse_s[TM], D_s[TM];
  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items_k, 1, it)) return;
  const int h = it.h, H = a.H, tid = threadIdx.x;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int j = it.tile * TN + tid;
  const bool kvalid = j < Lk;
  const int64_t krow = (int64_t)(kv0 + (kvalid ? j : 0)) * H + h;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    k[c] = kvalid ? ((const float*)a.K)[krow * D + c] : 0.0f;
    v[c] = kvalid ? ((const float*)a.V)[krow * D + c] : 0.0f;
    dk[c] = 0.0f;
    dv[c] = 0.0f;
  }
  const int win = a.win;
  const int nqt = win_end_qtile(min(Lk, (it.tile + 1) * TN) - 1, win, TM, (Lq + TM - 1) / TM);
  const int qt0 = CAUSAL ? (it.tile * TN) / TM : 0;
  for (int qt = qt0; qt < nqt; ++qt) {
    __syncthreads();
    load_tile_f32<D>(Qs, (const float*)a.Q, qt * TM, Lq, a.q_shared ? 0 : q0, H, h, tid);
    load_tile_f32<D>(dOs, (const float*)a.dO, qt * TM, Lq, q0, H, h, tid);
    {
      const int ii = qt * TM + tid;
      if (ACT == ACT_SOFTMAX && ii < Lq) {
        lse_s[tid] = a.lse[(int64_t)(q0 + ii) * H + h];
        D_s[tid] = a.Dvec[(int64_t)(q0 + ii) * H + h];
      } else {
        lse_s[tid] = 0.0f;
        D_s[tid] = 0.0f;
      }
    }
    __syncthreads();
    if (!kvalid) continue;
    for (int ii = 0; ii < TM; ++ii) {
      const int i = qt * TM + ii;
      if (i >= Lq || (CAUSAL && j > i) || (win > 0 && j <= i - win)) continue;
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s += Qs[ii][c] * k[c];
        dp += dOs[ii][c] * v[c];
      }
      s *= a.scale;
      if (BIAS) s += a.bias[(int64_t)h * a.nb + clampi(i - j, 0, a.nb - 1)];
      float p;
      const float ds = score_grad<ACT>(s, lse_s[ii], D_s[ii], dp, p);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        dk[c] += ds * Qs[ii][c];
        dv[c] += p * dOs[ii][c];
      }
    }
  }
  if (!kvalid) return;
  float* dkrow = (float*)a.dK + krow * D;
  float* dvrow = (float*)a.dV + krow * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    dkrow[c] = dk[c] * a.scale;
    dvrow[c] = dv[c];
  }
}

template <template <int, int, bool, bool> class KS, int D, int ACT>
struct Unused {};

#define GDPA_F32_DISPATCH(KERNEL, ARGS, GRID)                                                   \
  do {                                                                                         \
    const bool bias = p.nb > 0;                                                                \
    auto go = [&](auto dtag, auto atag, auto ctag, auto btag) {                                \
      constexpr int D_ = decltype(dtag)::value;                                                \
      constexpr int A_ = decltype(atag)::value;                                                \
      constexpr bool C_ = decltype(ctag)::value;                                               \
      constexpr bool B_ = decltype(btag)::value;                                               \
      hipLaunchKernelGGL((KERNEL<D_, A_, C_, B_>), dim3(GRID), dim3(64), 0, s, ARGS);         \
    };                                                                                         \
    auto with_cb = [&](auto dtag, auto atag) {                                                 \
      if (p.causal) {                                                                          \
        if (bias) go(dtag, atag, std::true_type{}, std::true_type{});                         \
        else go(dtag, atag, std::true_type{}, std::false_type{});                             \
      } else {                                                                                 \
        if (bias) go(dtag, atag, std::false_type{}, std::true_type{});                        \
        else go(dtag, atag, std::false_type{}, std::false_type{});                            \
      }                                                                                        \
    };                                                                                         \
    auto with_a = [&](auto dtag) {                                                             \
      if (p.act == ACT_SOFTMAX) with_cb(dtag, std::integral_constant<int, ACT_SOFTMAX>{});     \
      else if (p.act == ACT_GELU_TANH) with_cb(dtag, std::integral_constant<int, ACT_GELU_TANH>{}); \
      else with_cb(dtag, std::integral_constant<int, ACT_SILU>{});                             \
    };                                                                                         \
    if (p.D == 32) with_a(std::integral_constant<int, 32>{});                                  \
    else if (p.D == 64) with_a(std::integral_constant<int, 64>{});                             \
    else with_a(std::integral_constant<int, 128>{});                                           \
  } while (0)

}  // namespace

hipError_t launch_fwd_f32(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  GDPA_F32_DISPATCH(fwd_f32_kernel, a, grid);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const Prob& p, const BwdArgs& a, int grid_q, int grid_k, hipStream_t s) {
  if (grid_q > 0) GDPA_F32_DISPATCH(bwd_dq_f32_kernel, a, grid_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grid_k > 0) GDPA_F32_DISPATCH(bwd_dkdv_f32_kernel, a, grid_k);
  return hipGetLastError();
}

}  // namespace gdpa
