// Forward kernel template: JFA (softmax) and GDPA (GELU-tanh / SiLU), bf16 or MX-fp8 inputs,
// fp32 accumulation.
//
// Method (page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
// Model"): JFA paragraph - FlashAttention run directly on jagged tensors (no padding), with
// attention biases and different query / key lengths; GDPA paragraph - the same two products
// with an element-wise GELU or SiLU instead of softmax and no normalisation; low-precision part -
// attention with MXFP8 block-scaled matrix products. FlashAttention's tiling with online max /
// sum rescaling gives exactly the plain softmax result; GDPA needs no rescaling since every
// score is mapped on its own.
//
// Work decomposition: one workgroup (4 waves) per scheduler item = 128 query rows of one
// (sample, head). Each wave owns 32 queries. Keys stream through LDS in tiles of 64 rows; the
// global loads of the next tile (bf16: of the next two tiles, in two register stages) are
// issued before the current tile is computed.
//
// Operand choice (wave64 MFMA):
//   S^T = K Q^T  : A = K rows from LDS, B = Q^T from registers. The accumulator puts one query
//                  per lane (column) and 16 keys per lane (rows), so row statistics need only a
//                  swap between the two half-waves. bf16: 32x32x16 bf16 MFMA. MX: 32x32x64
//                  f8f6f4 scaled MFMA with e4m3 operands, whose per-32-element e8m0 scales run
//                  along D, the contraction dimension, so they are the instruction's own operand
//                  scales.
//   O^T += V^T P^T: A = V^T read transposed from the row-major bf16 V tile (ds_read_b64_tr_b16),
//                  B = P^T (bf16) straight from the S^T accumulator (the key order inside a
//                  16-key k-step is permuted identically on both operands). For MX, V is
//                  dequantised exactly into the bf16 tile by the scaled fp8 -> bf16 conversion
//                  instruction: an e4m3 value times a power of two has at most 4 significant
//                  bits. P is rounded to bf16 in both paths.
// The exp of softmax uses exp2 with log2(e) folded into the score scale.
#pragma once

#include <math.h>

#include "gdpa_common.h"
#include "gdpa_internal.h"
#include "gdpa_split.h"
#include "gdpa_tiles.h"

namespace gdpa {
namespace fwdk {

constexpr int BM = FWD_BM_BF16;  // queries per item (4 waves x 32)
constexpr int BN = FWD_BN_BF16;  // keys per tile
constexpr int NT = 256;

// 2^(X-127) for an e8m0 code X (0xFF, NaN in the format, is not produced by this path's inputs)
__device__ __forceinline__ float e8m0_value(uint32_t X) {
  return X == 0u ? 0x1p-127f : __builtin_bit_cast(float, X << 23);
}

template <int D, bool MX>
struct Smem {
  // MX K tile: 64 rows x 128 bytes, pitch 144 (16 rows of a read hit distinct bank groups),
  // then 64 scale words.
  static constexpr int KMX_P = 144;
  static constexpr int K_BYTES = MX ? BN * KMX_P + BN * 4 : Tile<D>::BYTES;
  static constexpr int V_BYTES = Tile<D>::BYTES;
  static constexpr int BIAS_BYTES = BIAS_WMAX * 4;
};

// WIN: causal sliding window of a.win keys (query i sees keys i - win + 1 .. i); bf16 only.
template <int D, int ACT, bool CAUSAL, bool BIAS, bool MX, bool WIN = false>
__global__ __launch_bounds__(NT, 2) void fwd_kernel(FwdArgs a) {
  static_assert(!MX || D == 128, "MX path is for D = 128");
  static_assert(!WIN || (CAUSAL && !MX), "windows are causal, bf16");
  using S = Smem<D, MX>;
  __shared__ __attribute__((aligned(16))) char smem[S::K_BYTES + S::V_BYTES + (BIAS ? S::BIAS_BYTES : 0)];
  GDPA_LDS char* Ks = (GDPA_LDS char*)smem;
  GDPA_LDS char* Vs = Ks + S::K_BYTES;
  GDPA_LDS float* bwin = (GDPA_LDS float*)(Vs + S::V_BYTES);
  __shared__ int flag_;

  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items, 0, it)) return;
  const int b = it.b, h = it.h, H = a.H;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int row_blk = it.tile * BM;   // first query of the item (local index)
  const int wrow = row_blk + w * 32;  // first query of this wave
  const int iq = wrow + l32;          // this lane's query
  const bool wave_active = wrow < Lq;
  const bool qv = iq < Lq;
  const int64_t qrow = (int64_t)(q0 + (qv ? iq : 0)) * H + h;  // O / lse row
  // Q row: in the sample's rows, or in the one block every sample shares
  const int64_t qin = a.q_shared ? (int64_t)(qv ? iq : 0) * H + h : qrow;

  int nkt = (Lk + BN - 1) / BN;
  if (CAUSAL) {
    const int i_max = min(Lq, row_blk + BM) - 1;
    nkt = min(nkt, i_max / BN + 1);
  }
  // key tiles of this item: all of them, or one chunk of a split tile (bf16 only), counted from
  // the first tile the item's sliding window reaches
  const int kt_first = WIN ? win_first_ktile(row_blk, a.win, BN) : 0;
  const int kt_lo = kt_first + it.lo, kt_hi = min(kt_first + it.hi, nkt);

  // ---- Q^T operand: lane holds query iq
  bf16x8 qop[MX ? 1 : D / 16];
  i32x8 q8[MX ? 2 : 1];
  uint32_t qsc = 0;
  if constexpr (!MX) {
    const __bf16* Q = (const __bf16*)a.Q;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qop[s] = qv ? *(const bf16x8*)(Q + qin * D + 16 * s + 8 * g) : zero_bf16x8();
  } else {
    const uint8_t* Q8 = (const uint8_t*)a.Q;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (qv) {
        lo = *(const i32x4*)(Q8 + qin * D + 64 * s + 16 * g);
        hi = *(const i32x4*)(Q8 + qin * D + 64 * s + 32 + 16 * g);
      }
      q8[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    qsc = qv ? *(const uint32_t*)(a.qs + qin * 4) : 0x7F7F7F7Fu;
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * a.nb : nullptr;
  // Bias window for this item over raw diagonals, reversed (bwin[t] = bias[clamp(w_hi - t)]) and
  // divided by scale, so that the 16 lookups of a lane are one base address plus constant
  // offsets and can seed the score accumulators.
  const float inv_scale = 1.0f / a.scale;  // the window holds bias / scale (see S^T below)
  int w_hi = 0;
  bool win_ok = false;

  // ---- global -> register staging of one K/V tile
  TileLoader<D, NT> lk_, lv_;           // bf16 path
  constexpr int MXC = BN * 128 / 16 / NT;  // 16-byte code chunks per thread (MX): 2
  i32x4 kc[MX ? MXC : 1], vc[MX ? MXC : 1];
  uint32_t ksw = 0, vsb[MX ? MXC : 1];
  auto load_tile = [&](int kt) {
    if constexpr (!MX) {
      lk_.load((const __bf16*)a.K, kt * BN, Lk, kv0, H, h, tid);
      lv_.load((const __bf16*)a.V, kt * BN, Lk, kv0, H, h, tid);
    } else {
      const uint8_t* K8 = (const uint8_t*)a.K;
      const uint8_t* V8 = (const uint8_t*)a.V;
#pragma unroll
      for (int u = 0; u < MXC; ++u) {
        const int c = tid + NT * u, r = c >> 3, col = c & 7;
        const int j = kt * BN + r;
        if (j < Lk) {
          const int64_t off = ((int64_t)(kv0 + j) * H + h) * 128 + col * 16;
          kc[u] = *(const i32x4*)(K8 + off);
          vc[u] = *(const i32x4*)(V8 + off);
          vsb[u] = a.vs[((int64_t)(kv0 + j) * H + h) * 4 + (col >> 1)];
        } else {
          kc[u] = i32x4{0, 0, 0, 0};
          vc[u] = i32x4{0, 0, 0, 0};
          vsb[u] = 127u;
        }
      }
      if (tid < BN) {
        const int j = kt * BN + tid;
        ksw = j < Lk ? *(const uint32_t*)(a.ks + ((int64_t)(kv0 + j) * H + h) * 4) : 0x7F7F7F7Fu;
      }
    }
  };
  auto store_tile = [&]() {
    if constexpr (!MX) {
      lk_.store(Ks, tid);
      lv_.store(Vs, tid);
    } else {
#pragma unroll
      for (int u = 0; u < MXC; ++u) {
        const int c = tid + NT * u, r = c >> 3, col = c & 7;
        *(GDPA_LDS i32x4*)(Ks + r * S::KMX_P + col * 16) = kc[u];
        // dequantise 16 V codes into two 16-byte bf16 chunks: each conversion takes two e4m3
        // bytes of a word (low or high half) times the block's power-of-two scale; the products
        // have at most 4 significant bits, so bf16 holds them exactly
        const float sc = e8m0_value(vsb[u]);
        bf16x2 pv[8];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          pv[2 * wd] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vc[u][wd], sc, false);
          pv[2 * wd + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vc[u][wd], sc, true);
        }
        const bf16x8 lo8 = {pv[0][0], pv[0][1], pv[1][0], pv[1][1], pv[2][0], pv[2][1], pv[3][0], pv[3][1]};
        const bf16x8 hi8 = {pv[4][0], pv[4][1], pv[5][0], pv[5][1], pv[6][0], pv[6][1], pv[7][0], pv[7][1]};
        *(GDPA_LDS bf16x8*)(Vs + Tile<D>::off(r, col * 16)) = lo8;
        *(GDPA_LDS bf16x8*)(Vs + Tile<D>::off(r, col * 16 + 8)) = hi8;
      }
      if (tid < BN) *(GDPA_LDS uint32_t*)(Ks + BN * S::KMX_P + tid * 4) = ksw;
    }
  };

  if (kt_lo < kt_hi) load_tile(kt_lo);
  if (BIAS && kt_lo < kt_hi) {  // staged while the first tile's loads are in flight
    // raw diagonals iq - j of the item: iq in [row_blk, row_blk + BM), j in its key tiles
    w_hi = row_blk + BM - 1 - kt_lo * BN;
    win_ok = __builtin_amdgcn_readfirstlane((int)stage_bias_window(
                 bwin, bias_h, a.nb, row_blk - (kt_hi * BN - 1), w_hi, true, inv_scale, tid, NT)) != 0;
  }
  // one key tile: scores, probabilities and the P.V products, from the tile in LDS
  auto compute = [&](int kt) {
    const int k0 = kt * BN;
    if (!wave_active) return;
    if (CAUSAL && k0 > wrow + 31) return;  // every key of the tile is after every query
    if (WIN && k0 + BN <= wrow - a.win + 1) return;  // ... or before every query's window

    // ---- S^T = K Q^T for two 32-key blocks. With a bias the accumulators start from
    // bias / scale read straight from the LDS window (register r of block kb is key
    // j = k0 + kb*32 + (r/4)*8 + 4g + r%4, diagonal iq - j), so the products land on top of it.
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
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!MX) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          sacc[kb] = mfma32(tile_row_op<D>(Ks, kb * 32, s, lane), qop[s], sacc[kb]);
      } else {
        const int r = kb * 32 + l32;
        const uint32_t kw = *(const GDPA_LDS uint32_t*)(Ks + BN * S::KMX_P + r * 4);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x4 lo = *(const GDPA_LDS i32x4*)(Ks + r * S::KMX_P + 64 * s + 16 * g);
          const i32x4 hi = *(const GDPA_LDS i32x4*)(Ks + r * S::KMX_P + 64 * s + 32 + 16 * g);
          const i32x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          // this lane supplies the scale of its row for k block g of the instruction, which is
          // the 32-element block 2s + g along D
          const int sa = (int)((kw >> (8 * (2 * s + g))) & 0xFFu);
          const int sb = (int)((qsc >> (8 * (2 * s + g))) & 0xFFu);
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, q8[s], sacc[kb], 0, 0, 0,
                                                                     sa, 0, sb);
        }
      }
    }

    // ---- scores -> probabilities. Masking is needed only on tiles that reach past the keys,
    // past the wave's first query (causal) or before its last query's window; valid keys of
    // block kb satisfy lo_kb <= (r/4)*8 + 4g + r%4 < lim_kb.
    const bool need_mask = __builtin_amdgcn_readfirstlane(
        (int)((k0 + BN > Lk) || (CAUSAL && k0 + BN - 1 > wrow) || (WIN && k0 < wrow + 32 - a.win))) != 0;
    int lim[2], lo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int l = Lk - (k0 + kb * 32);
      if (CAUSAL) l = min(l, iq - (k0 + kb * 32) + 1);
      lim[kb] = l - 4 * g;
      lo[kb] = WIN ? iq - a.win + 1 - (k0 + kb * 32) - 4 * g : -64;
    }
    auto masked = [&](int kb, int r) {
      const int off = (r >> 2) * 8 + (r & 3);
      return off >= lim[kb] || (WIN && off < lo[kb]);
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
      // row max on the raw accumulators (scale > 0 preserves order), then one fma + exp2
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
      mt = half_max(mt) * sl2;
      // The reference maximum m_run moves only when a row's maximum exceeds it by more than 8
      // (log2 units), so probabilities stay below 2^8 and the running output is rescaled
      // rarely; the final normalisation uses the same reference, so the result is unchanged.
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
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb][r] = fast_exp2(fmaf(sacc[kb][r], sl2, -m_use));
          ls += p[kb][r];
        }
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

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(&p[kb][8 * s2]);
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
          o[n] = mfma32(tile_tr_op<D>(Vs, kb * 32 + 16 * s2, n, lane), pb, o[n]);
      }
    }
  };
  if constexpr (MX) {
    // one tile in flight in registers while the previous one is computed
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
      __syncthreads();
      store_tile();
      __syncthreads();
      if (kt + 1 < kt_hi) load_tile(kt + 1);
      compute(kt);
    }
  } else {
    // bf16: two tiles in flight in two register stages (A: even offsets from kt_lo, B: odd),
    // which doubles the bytes a workgroup has in flight; short query blocks (one busy wave, as
    // in PMA) are bound by exactly that
    TileLoader<D, NT> lk2_, lv2_;
    if (kt_lo + 1 < kt_hi) {
      lk2_.load((const __bf16*)a.K, (kt_lo + 1) * BN, Lk, kv0, H, h, tid);
      lv2_.load((const __bf16*)a.V, (kt_lo + 1) * BN, Lk, kv0, H, h, tid);
    }
    for (int kt = kt_lo; kt < kt_hi; kt += 2) {
      __syncthreads();
      store_tile();
      __syncthreads();
      if (kt + 2 < kt_hi) load_tile(kt + 2);
      compute(kt);
      if (kt + 1 < kt_hi) {
        __syncthreads();
        lk2_.store(Ks, tid);
        lv2_.store(Vs, tid);
        __syncthreads();
        if (kt + 3 < kt_hi) {
          lk2_.load((const __bf16*)a.K, (kt + 3) * BN, Lk, kv0, H, h, tid);
          lv2_.load((const __bf16*)a.V, (kt + 3) * BN, Lk, kv0, H, h, tid);
        }
        compute(kt + 1);
      }
    }
  }

  if (!MX && it.slot >= 0) {
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
      split::combine_fwd_tile<ACT == ACT_SOFTMAX, D>(a, b, it.tile, h, n, first);
    return;
  }
  if (!wave_active) return;
  // ---- epilogue: lane owns query iq; register r of block n is d = n*32 + (r/4)*8 + 4g + r%4
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

template <int D, int ACT, bool CAUSAL, bool BIAS, bool MX, bool WIN = false>
hipError_t launch_t(const FwdArgs& a, int grid, hipStream_t s) {
  prof_before(PROF_FWD, s);
  hipLaunchKernelGGL((fwd_kernel<D, ACT, CAUSAL, BIAS, MX, WIN>), dim3(grid), dim3(NT), 0, s, a);
  prof_after(PROF_FWD, s);
  return hipGetLastError();
}

template <int D, int ACT, bool MX>
hipError_t launch_cb(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  const bool bias = p.nb > 0;
  if constexpr (!MX) {
    if (p.win > 0)
      return bias ? launch_t<D, ACT, true, true, false, true>(a, grid, s)
                  : launch_t<D, ACT, true, false, false, true>(a, grid, s);
  }
  if (p.causal)
    return bias ? launch_t<D, ACT, true, true, MX>(a, grid, s) : launch_t<D, ACT, true, false, MX>(a, grid, s);
  return bias ? launch_t<D, ACT, false, true, MX>(a, grid, s) : launch_t<D, ACT, false, false, MX>(a, grid, s);
}

template <int D, bool MX>
hipError_t launch_d(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_cb<D, ACT_SOFTMAX, MX>(p, a, grid, s);
    case ACT_GELU_TANH: return launch_cb<D, ACT_GELU_TANH, MX>(p, a, grid, s);
    default: return launch_cb<D, ACT_SILU, MX>(p, a, grid, s);
  }
}

}  // namespace fwdk
}  // namespace gdpa
