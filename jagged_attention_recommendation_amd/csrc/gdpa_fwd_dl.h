// Forward kernel for D = 128 bf16 with direct global -> LDS tile loads and a two-stage LDS ring.
//
// Same method and operand orientation as gdpa_fwd_kernel.h (JFA softmax / GDPA activation on
// jagged tensors, page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
// Foundation Model", JFA and GDPA paragraphs). What differs is the data movement: K and V tiles
// (64 keys x 256 bytes, layout in gdpa_dl.h) are fetched with direct loads, and while a tile is
// computed the next one streams into the other stage; one barrier per tile.
#pragma once

#include <math.h>

#include "gdpa_common.h"
#include "gdpa_dl.h"
#include "gdpa_internal.h"
#include "gdpa_split.h"
#include "gdpa_tiles.h"  // store_acc_row_bf16

namespace gdpa {
namespace fwddl {

using namespace dl;

constexpr int BM = FWD_BM_BF16;  // queries per item (4 waves x 32)
constexpr int BN = FWD_BN_BF16;  // keys per tile
static_assert(BN == ROWS, "one key tile is one direct-load tile");
constexpr int NT = 256;
constexpr int WMAX = 3072;        // bias window (floats) staged in LDS

// WIN: causal sliding window of a.win keys (query i sees keys i - win + 1 .. i).
template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
__global__ __launch_bounds__(NT, 2) void fwd_dl_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char sk0_[TILE];
  __shared__ __attribute__((aligned(16))) char sv0_[TILE];
  __shared__ __attribute__((aligned(16))) char sk1_[TILE];
  __shared__ __attribute__((aligned(16))) char sv1_[TILE];
  __shared__ __attribute__((aligned(16))) float bwin_[BIAS ? WMAX : 1];
  __shared__ int flag_;
  GDPA_LDS char* sk0 = (GDPA_LDS char*)sk0_;
  GDPA_LDS char* sv0 = (GDPA_LDS char*)sv0_;
  GDPA_LDS char* sk1 = (GDPA_LDS char*)sk1_;
  GDPA_LDS char* sv1 = (GDPA_LDS char*)sv1_;
  GDPA_LDS float* bwin = (GDPA_LDS float*)bwin_;

  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items, 0, it)) return;
  const int b = it.b, h = it.h, H = a.H;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_blk = it.tile * BM;
  const int wrow = row_blk + w * 32;
  const int iq = wrow + l32;
  const bool wave_active = wrow < Lq;
  const bool qv = iq < Lq;
  const int64_t qrow = (int64_t)(q0 + (qv ? iq : 0)) * H + h;  // O / lse row

  int nkt = (Lk + BN - 1) / BN;
  if (CAUSAL) nkt = min(nkt, (min(Lq, row_blk + BM) - 1) / BN + 1);
  // key tiles of this item: all of them, or one chunk of a split tile, counted from the first
  // tile the item's sliding window reaches
  const int kt_first = WIN ? win_first_ktile(row_blk, a.win, BN) : 0;
  const int kt_lo = kt_first + it.lo, kt_hi = min(kt_first + it.hi, nkt);

  // The item's query rows come in as direct-load tiles (whole cache lines per instruction) into
  // stage 1, idle until the second key tile: rows row_blk .. + 63, then row_blk + 64 .. + 127,
  // of the sample or of the one block every sample shares.
  {
    const __bf16* Q = (const __bf16*)a.Q;
    const int qbase = a.q_shared ? 0 : q0;
    issue_tile(sk1, Q, row_blk, Lq, qbase, H, h, w, lane);
    if (Lq > row_blk + ROWS) issue_tile(sv1, Q, row_blk + ROWS, Lq, qbase, H, h, w, lane);
  }
  // The bias window (raw diagonals iq - j: iq in the item, j in its key tiles) comes in the same
  // way, bwin[t] = bias[clamp(w_hi - t)], and is scaled by 1 / scale after the wait.
  const float* bias_h = BIAS ? a.bias + (int64_t)h * a.nb : nullptr;
  int w_hi = 0, wcnt = 0;
  if (BIAS && kt_lo < kt_hi) {
    w_hi = row_blk + BM - 1 - kt_lo * BN;
    wcnt = w_hi - (row_blk - (kt_hi * BN - 1)) + 1;
    if (wcnt > WMAX) wcnt = 0;  // too wide to stage: looked up in the table instead
    issue_window(bwin, bias_h, a.nb, w_hi, -1, wcnt, w, lane);
  }
  const bool win_ok = wcnt > 0;
  const __bf16* K = (const __bf16*)a.K;
  const __bf16* V = (const __bf16*)a.V;
  if (kt_lo < kt_hi) {
    issue_tile(sk0, K, kt_lo * BN, Lk, kv0, H, h, w, lane);
    issue_tile(sv0, V, kt_lo * BN, Lk, kv0, H, h, w, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's row and window loads have landed
  __syncthreads();                // ... and everyone else's
  // wave w's 32 rows: tile w / 2, rows 32 (w % 2) ..; a wave past the item's rows uses zeros
  bf16x8 qop[D / 16];
  {
    const GDPA_LDS char* tq = (w >> 1) ? sv1 : sk1;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = wave_active ? row_op(tq, (w & 1) * 32, s, lane) : zero_bf16x8();
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = a.scale * LOG2E;
  const float inv_scale = 1.0f / a.scale;
  if (win_ok)  // read at the first key tile, after its barrier
    for (int t = tid; t < wcnt; t += NT) bwin[t] *= inv_scale;

  // one key tile: scores, probabilities, output update (stage buffers passed in)
  auto tile = [&](const GDPA_LDS char* __restrict__ Ks, const GDPA_LDS char* __restrict__ Vs, int k0) {
    f32x16 sacc[2];
    if (BIAS && win_ok) {
      const GDPA_LDS float* bp = bwin + (w_hi - iq + k0 + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = bp[kb * 32 + (r >> 2) * 8 + (r & 3)];
    } else if (BIAS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[kb][r] = bias_h[clampi(iq - (k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3)), 0, a.nb - 1)] * inv_scale;
    } else {
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) sacc[kb] = mfma32(row_op(Ks, kb * 32, s, lane), qop[s], sacc[kb]);

    const bool need_mask = __builtin_amdgcn_readfirstlane(
        (int)((k0 + BN > Lk) || (CAUSAL && k0 + BN - 1 > wrow) || (WIN && k0 < wrow + 32 - a.win))) != 0;
    // register r of half kb (key offset o = 8 (r / 4) + r % 4) is valid for lo[kb] <= o < lim[kb]
    int lim[2], lo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int l = Lk - (k0 + kb * 32);
      if (CAUSAL) l = min(l, iq - (k0 + kb * 32) + 1);
      lim[kb] = l - 4 * g;
      lo[kb] = WIN ? iq - a.win + 1 - (k0 + kb * 32) - 4 * g : -64;
    }
    auto masked = [&](int kb, int r) {
      const int o = (r >> 2) * 8 + (r & 3);
      return o >= lim[kb] || (WIN && o < lo[kb]);
    };
    float p[2][16];
    if (ACT == ACT_SOFTMAX) {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (masked(kb, r)) sacc[kb][r] = -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
      mt = half_max(mt) * sl2;
      const bool grow = mt > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : m_run;
        const float alpha = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) o[n] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.0f : m_run;
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb][r] = fast_exp2(fmaf(sacc[kb][r], sl2, -m_use));
          ls += p[kb][r];
        }
      l_run += ls;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = act_fwd(ACT, sacc[kb][r] * a.scale);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (masked(kb, r)) p[kb][r] = 0.0f;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(&p[kb][8 * s2]);
#pragma unroll
        for (int n = 0; n < D / 32; ++n) o[n] = mfma32(tr_op(Vs, kb * 32 + 16 * s2, n, lane), pb, o[n]);
      }
  };

  // whether this wave computes key tile kt: not wholly after its last query (causal) nor wholly
  // before its first query's window
  auto wave_needs = [&](int kt) {
    return wave_active && !(CAUSAL && kt * BN > wrow + 31) && !(WIN && (kt + 1) * BN <= wrow - a.win + 1);
  };
  // Two stages, loop unrolled by two so each stage is a distinct LDS object: the direct loads
  // into one stage can then stay in flight while the other stage is read.
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads for tile kt have landed
    __syncthreads();                // ... and everyone else's; tile kt - 1 is done with stage 1
    if (kt + 1 < kt_hi) {
      issue_tile(sk1, K, (kt + 1) * BN, Lk, kv0, H, h, w, lane);
      issue_tile(sv1, V, (kt + 1) * BN, Lk, kv0, H, h, w, lane);
    }
    if (wave_needs(kt)) tile(sk0, sv0, kt * BN);
    if (kt + 1 >= kt_hi) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 2 < kt_hi) {
      issue_tile(sk0, K, (kt + 2) * BN, Lk, kv0, H, h, w, lane);
      issue_tile(sv0, V, (kt + 2) * BN, Lk, kv0, H, h, w, lane);
    }
    if (wave_needs(kt + 1)) tile(sk1, sv1, (kt + 1) * BN);
  }

  if (it.slot >= 0) {
    // chunk of a split tile: unnormalised output rows and, for softmax, the running max (log2
    // units) and sum; the workgroup that completes the tile combines its chunks in order
    if (wave_active) {
      float* po = a.part_o + ((int64_t)it.slot * BM + w * 32 + l32) * D;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(po + n * 32 + r4 * 8 + 4 * g) =
              f32x4{o[n][4 * r4], o[n][4 * r4 + 1], o[n][4 * r4 + 2], o[n][4 * r4 + 3]};
      if (ACT == ACT_SOFTMAX) {
        const float lt = half_sum(l_run);
        if (g == 0) {
          float* pml = a.part_ml + (int64_t)it.slot * 2 * BM;
          pml[w * 32 + l32] = m_run;
          pml[BM + w * 32 + l32] = lt;
        }
      }
    }
    const int first = it.slot - split::chunk_index(it.chunk), n = split::chunk_count(it.chunk);
    if (split::chunk_done(a.split_cnt + first, n, (GDPA_LDS int*)&flag_))
      split::combine_fwd_tile<ACT == ACT_SOFTMAX>(a, b, it.tile, h, n, first);
    return;
  }
  if (!wave_active) return;
  float inv = 1.0f;
  if (ACT == ACT_SOFTMAX) {
    const float lt = half_sum(l_run);
    inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qv && g == 0 && a.lse != nullptr)
      a.lse[qrow] = lt > 0.0f ? (m_run + log2f(lt)) * LN2 : -INFINITY;
  }
  if (!qv) return;
  __bf16* orow = (__bf16*)a.O + qrow * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) store_acc_row_bf16(orow, o[n], n, g, inv);
}

template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
hipError_t launch_t(const FwdArgs& a, int grid, hipStream_t s) {
  prof_before(PROF_FWD, s);
  hipLaunchKernelGGL((fwd_dl_kernel<ACT, CAUSAL, BIAS, WIN>), dim3(grid), dim3(NT), 0, s, a);
  prof_after(PROF_FWD, s);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_cb(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  const bool bias = p.nb > 0;
  if (p.win > 0) return bias ? launch_t<ACT, true, true, true>(a, grid, s) : launch_t<ACT, true, false, true>(a, grid, s);
  if (p.causal) return bias ? launch_t<ACT, true, true>(a, grid, s) : launch_t<ACT, true, false>(a, grid, s);
  return bias ? launch_t<ACT, false, true>(a, grid, s) : launch_t<ACT, false, false>(a, grid, s);
}

inline hipError_t launch(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_cb<ACT_SOFTMAX>(p, a, grid, s);
    case ACT_GELU_TANH: return launch_cb<ACT_GELU_TANH>(p, a, grid, s);
    default: return launch_cb<ACT_SILU>(p, a, grid, s);
  }
}

}  // namespace fwddl
}  // namespace gdpa
