// Backward kernels, bf16 inputs, fp32 accumulation, for JFA (softmax) and GDPA (GELU-tanh/SiLU).
//
// Method (page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
// Model"): the JFA paragraph asks for efficient backward passes on jagged tensors; the GDPA
// paragraph gives the forward as act(QK^T)V; the block-attention paragraph names the two extra
// costs of the softmax backward, the stored logsumexp and the row term Di. The backward
// recomputes the scores instead of storing them:
//   p_ij  = exp(s_ij - lse_i)                (softmax)    or act(s_ij)              (GDPA)
//   dp_ij = <do_i, v_j>
//   ds_ij = p_ij (dp_ij - D_i), D_i = <do_i, o_i>      or dp_ij * act'(s_ij)
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,   dbias[h, clamp(i-j)] += ds_ij
//
// Two kernels, so every output row is written by exactly one work item and nothing is
// accumulated with atomics (results are bitwise reproducible):
//   dq_kernel   : item = 128 queries of one (sample, head); loops over key tiles. Also computes
//                 D_i (softmax) and the item's diagonal sums of dS for the bias gradient.
//   dkdv_kernel : item = 128 keys of one (sample, head); loops over query tiles.
// MFMA operand choices (32x32x16 bf16), with the accumulator layout noted in gdpa_common.h:
//   dq_kernel   S^T = K Q^T, dP^T = V dO^T (lane = query); dQ^T += K^T dS^T with K^T read
//               transposed from the K tile.
//   dkdv_kernel S = Q K^T, dP = dO V^T (lane = key); dV^T += dO^T P and dK^T += Q^T dS with
//               dO^T and Q^T read transposed from the query tiles.
#include <math.h>

#include "gdpa_bwd_dl.h"
#include "gdpa_common.h"
#include "gdpa_internal.h"
#include "gdpa_split.h"
#include "gdpa_tiles.h"

namespace gdpa {

namespace {

constexpr int NT = 256;         // threads per workgroup (4 waves)
constexpr int QI = BWD_Q_ITEM;  // queries per dQ item
constexpr int KL = BWD_K_LOOP;  // keys per tile in the dQ loop
constexpr int KI = BWD_K_ITEM;  // keys per dK/dV item
constexpr int QL = BWD_Q_LOOP;  // queries per tile in the dK/dV loop
static_assert(QI == 128 && KI == 128 && KL == 64 && QL == 64, "kernels assume these tiles");

template <int ACT>
__device__ __forceinline__ float dscore(float s2, float s, float lse2, float Di, float dp, float& p) {
  // s2: score in log2 units (softmax), s: natural score (GDPA)
  if (ACT == ACT_SOFTMAX) {
    p = fast_exp2(s2 - lse2);
    return p * (dp - Di);
  }
  float y, dy;
  act_fwd_bwd(ACT, s, y, dy);
  p = y;
  return dp * dy;
}

// ------------------------------------------------------------------------------------------
// dQ
//
// Bias gradient inside this kernel. A wave's 32 x 64 block of dS (queries a, keys c) has 95
// diagonals d = a - c in [-63, 31]. The wave writes the block to its own LDS buffer, then every
// lane sums exactly 32 elements: lane 31 + t (t = 0..32) the full diagonal d = t - 32, and lane
// t < 31 the two short diagonals d = t - 63 and d = t + 1. A diagonal with d < -32 continues in
// the next key tile as d + 64 - the same lane's second diagonal - so lane t keeps it in a
// register and adds it there. After each tile the 64 diagonals that no later tile reaches are
// complete and are written once to the wave's partial row in global memory. Every sum is formed
// in a fixed order; diagonals that clamp to the table's ends are combined by a fixed-order wave
// reduction.
constexpr int DSP = 68;  // floats per row of a wave's dS buffer (16-byte aligned rows)

// WIN: causal sliding window of a.win keys (query i sees keys i - win + 1 .. i).
template <int D, int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
__global__ __launch_bounds__(NT, 1) void dq_kernel(BwdArgs a) {
  using T = Tile<D>;
  constexpr int BIAS_BYTES = BIAS ? BIAS_WMAX * 4 + 4 * 32 * DSP * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BYTES + BIAS_BYTES];
  GDPA_LDS char* Ks = (GDPA_LDS char*)smem;
  GDPA_LDS char* Vs = Ks + T::BYTES;
  GDPA_LDS float* bwin = (GDPA_LDS float*)(Vs + T::BYTES);
  GDPA_LDS float* dsbuf_all = bwin + BIAS_WMAX;  // [wave][32][DSP]
  __shared__ int flag_;

  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items_q, 0, it)) return;
  const int b = it.b, h = it.h, H = a.H, nb = a.nb;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int i0 = it.tile * QI;
  const int wrow = i0 + w * 32;
  const int iq = wrow + l32;
  const bool qv = iq < Lq;
  const bool wave_active = wrow < Lq;
  const int64_t row = (int64_t)(q0 + (qv ? iq : 0)) * H + h;  // O, dO, lse, D row
  // Q row: in the sample's rows, or in the one block every sample shares
  const int64_t qin = a.q_shared ? (int64_t)(qv ? iq : 0) * H + h : row;

  const __bf16* Q = (const __bf16*)a.Q;
  const __bf16* dO = (const __bf16*)a.dO;

  bf16x8 qop[D / 16], doop[D / 16];
  float part_d = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qop[s] = qv ? *(const bf16x8*)(Q + qin * D + 16 * s + 8 * g) : zero_bf16x8();
    doop[s] = qv ? *(const bf16x8*)(dO + row * D + 16 * s + 8 * g) : zero_bf16x8();
    if (ACT == ACT_SOFTMAX && qv) {
      const bf16x8 ov = *(const bf16x8*)((const __bf16*)a.O + row * D + 16 * s + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) part_d += (float)doop[s][e] * (float)ov[e];
    }
  }
  float Di = 0.0f, lse2 = 0.0f;
  if (ACT == ACT_SOFTMAX) {
    Di = half_sum(part_d);
    if (qv) {
      lse2 = a.lse[row] * LOG2E;
      // every chunk of a split tile computes it; the first writes it
      if (g == 0 && split::chunk_index(it.chunk) == 0) a.Dvec[row] = Di;
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) dq[n] = f32x16{};

  int nkt = (Lk + KL - 1) / KL;
  if (CAUSAL) nkt = min(nkt, (min(Lq, i0 + QI) - 1) / KL + 1);
  if (i0 >= Lq) nkt = 0;
  // key tiles of this item: all of them, or one chunk of a split tile (splitting is used only
  // without a bias table, whose partial rows assume whole tiles), counted from the first tile
  // the item's sliding window reaches
  const int kt_first = WIN ? win_first_ktile(i0, a.win, KL) : 0;
  const int kt_lo = kt_first + it.lo, kt_hi = min(kt_first + it.hi, nkt);

  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;
  const float bmul = ACT == ACT_SOFTMAX ? LOG2E : 1.0f;
  int w_hi = 0;
  bool win_ok = false;
  GDPA_LDS float* dsbuf = dsbuf_all + w * 32 * DSP;
  float carry = 0.0f;  // lanes t < 31: partial sum of diagonal t - 63 of the previous tile
  float* part = nullptr;
  float e_lo = 0.0f, e_hi = 0.0f;
  bool has_lo = false, has_hi = false;
  if (BIAS) {
    part = a.dbias_part + ((int64_t)h * a.part_rows + it.aux * (QI / 32) + w) * nb;
  }
  // Writes the complete diagonal d of this wave (value v) to its partial row; the ends of the
  // table collect every diagonal that clamps to them, summed over the wave in a fixed order.
  // Under causal masking diagonals d < 0 hold only masked (zero) entries and are skipped.
  auto emit = [&](int d, float v, bool valid) {
    if (CAUSAL && d < 0) valid = false;
    const bool lo = valid && d <= 0;
    const bool hi = valid && !lo && d >= nb - 1;
    if (valid && !lo && !hi) part[d] = v;
    const uint64_t blo = __builtin_amdgcn_ballot_w64(lo), bhi = __builtin_amdgcn_ballot_w64(hi);
    if (blo != 0) {
      e_lo += wave_sum(lo ? v : 0.0f);
      has_lo = true;
    }
    if (bhi != 0) {
      e_hi += wave_sum(hi ? v : 0.0f);
      has_hi = true;
    }
  };
  int k0_last = -1;

  TileLoader<D, NT> lk_, lv_;
  if (kt_lo < kt_hi) {
    lk_.load((const __bf16*)a.K, kt_lo * KL, Lk, kv0, H, h, tid);
    lv_.load((const __bf16*)a.V, kt_lo * KL, Lk, kv0, H, h, tid);
  }
  if (BIAS && kt_lo < kt_hi) {  // staged while the first tile's loads are in flight
    // raw diagonals iq - j: iq in [i0, i0 + QI), j in the item's key tiles
    w_hi = i0 + QI - 1 - kt_lo * KL;
    win_ok = __builtin_amdgcn_readfirstlane((int)stage_bias_window(
                 bwin, bias_h, nb, i0 - (kt_hi * KL - 1), w_hi, true, bmul, tid, NT)) != 0;
  }
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    __syncthreads();
    lk_.store(Ks, tid);
    lv_.store(Vs, tid);
    __syncthreads();
    if (kt + 1 < kt_hi) {
      lk_.load((const __bf16*)a.K, (kt + 1) * KL, Lk, kv0, H, h, tid);
      lv_.load((const __bf16*)a.V, (kt + 1) * KL, Lk, kv0, H, h, tid);
    }
    const int k0 = kt * KL;
    // the wave's tiles: not wholly after its last query (causal) nor wholly before its first
    // query's window (the bias-gradient reduction assumes the same range)
    if (!wave_active || (CAUSAL && k0 > wrow + 31) || (WIN && k0 + KL <= wrow - a.win + 1)) continue;
    k0_last = k0;
    f32x16 ds_acc[2], dp_acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ds_acc[kb] = f32x16{};
      dp_acc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        ds_acc[kb] = mfma32(tile_row_op<D>(Ks, kb * 32, s, lane), qop[s], ds_acc[kb]);
        dp_acc[kb] = mfma32(tile_row_op<D>(Vs, kb * 32, s, lane), doop[s], dp_acc[kb]);
      }
    }
    const bool need_mask = (k0 + KL > Lk) || (CAUSAL && k0 + KL - 1 > wrow) || (WIN && k0 < wrow + 32 - a.win);
    // scores in place: x = s * scale (* log2 e for softmax) + bias of diagonal iq - j
    const float sc = ACT == ACT_SOFTMAX ? sl2 : a.scale;
    if (BIAS) {
      if (win_ok) {
        const GDPA_LDS float* bp = bwin + (w_hi - iq + k0 + 4 * g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ds_acc[kb][r] = ds_acc[kb][r] * sc + bp[kb * 32 + (r >> 2) * 8 + (r & 3)];
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ds_acc[kb][r] = ds_acc[kb][r] * sc +
                            bias_h[clampi(iq - (k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3)), 0, nb - 1)] * bmul;
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ds_acc[kb] *= sc;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
        const float x = ds_acc[kb][r];
        float p;
        float ds = dscore<ACT>(x, x, lse2, Di, dp_acc[kb][r], p);
        if (!qv || (need_mask && (j >= Lk || (CAUSAL && j > iq) || (WIN && j <= iq - a.win)))) ds = 0.0f;
        ds_acc[kb][r] = ds;
      }
    }
    if (BIAS) {
      // dS block -> LDS (row = query a, column = key c; registers 4m..4m+3 are 4 consecutive keys)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 v4 = {ds_acc[kb][4 * m], ds_acc[kb][4 * m + 1], ds_acc[kb][4 * m + 2],
                            ds_acc[kb][4 * m + 3]};
          *(GDPA_LDS f32x4*)(dsbuf + l32 * DSP + kb * 32 + m * 8 + 4 * g) = v4;
        }
    }
    // dS^T as bf16 B operands (registers 8*s2..8*s2+7 of block kb), then dQ^T += K^T dS^T
    bf16x8 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = ds_acc[kb][8 * s2 + e];
        dsb[kb][s2] = pack8(tmp);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
          dq[n] = mfma32(tile_tr_op<D>(Ks, kb * 32 + 16 * s2, n, lane), dsb[kb][s2], dq[n]);
    if (BIAS) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Lane 31 + t sums diagonal t - 32 (rows 0..31); lane t < 31 sums diagonal t - 63 (rows
      // 0..t) and then diagonal t + 1 (rows t + 1..31). In both cases step s reads row s,
      // column (s + 63 - lane) mod 64, and the second diagonal starts where the column wraps.
      // All 64 lanes read one row at distinct columns: no bank conflicts.
      float s_a = 0.0f, s_b = 0.0f;
#pragma unroll
      for (int a8 = 0; a8 < 32; a8 += 8) {  // 8 reads in flight, then their sums
        float vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = dsbuf[(a8 + e) * DSP + ((a8 + e + 63 - lane) & 63)];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (a8 + e + 63 - lane < 64) s_a += vv[e]; else s_b += vv[e];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // complete after this tile: lanes t < 31 emit d = t + 1 (with the carried part), the
      // others emit d = lane - 63; absolute diagonal = wrow - k0 + d
      float v;
      int dabs;
      if (lane < 31) {
        v = carry + s_b;
        carry = s_a;
        dabs = wrow - k0 + lane + 1;
      } else {
        v = s_a;
        dabs = wrow - k0 + lane - 63;
      }
      emit(dabs, v, true);
    }
  }
  if (BIAS && k0_last >= 0) {
    // the 31 carried diagonals d = t - 63 of the last tile
    emit(wrow - k0_last + lane - 63, carry, lane < 31);
    if (lane == 0) {
      if (nb == 1) {
        if (has_lo || has_hi) part[0] = e_lo + e_hi;
      } else {
        if (has_lo) part[0] = e_lo;
        if (has_hi) part[nb - 1] = e_hi;
      }
    }
  }
  if (!BIAS && it.slot >= 0) {
    // chunk of a split tile: fp32 partial rows; the workgroup that completes the tile combines
    // its chunks in order
    if (wave_active) {
      float* pq = a.part_dq + ((int64_t)it.slot * QI + w * 32 + l32) * D;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(pq + n * 32 + r4 * 8 + 4 * g) =
              f32x4{dq[n][4 * r4], dq[n][4 * r4 + 1], dq[n][4 * r4 + 2], dq[n][4 * r4 + 3]};
    }
    const int first = it.slot - split::chunk_index(it.chunk), n = split::chunk_count(it.chunk);
    if (split::chunk_done(a.split_cnt_q + first, n, (GDPA_LDS int*)&flag_))
      split::combine_dq_tile<D>(a, b, it.tile, h, n, first);
    return;
  }
  if (!qv) return;
  if (a.dq_f32) {  // shared Q: this sample's gradient, summed over samples afterwards
#pragma unroll
    for (int n = 0; n < D / 32; ++n) store_acc_row_f32(a.dq_f32 + row * D, dq[n], n, g, a.scale);
    return;
  }
  __bf16* dqrow = (__bf16*)a.dQ + row * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) store_acc_row_bf16(dqrow, dq[n], n, g, a.scale);
}

// ------------------------------------------------------------------------------------------
// dK, dV
// Three workgroups per compute unit at D = 32 (their item count is large and each item short);
// at D = 64 the third does not fit without spills.
// WIN: causal sliding window of a.win keys (key j is seen by queries j .. j + win - 1).
template <int D, int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
__global__ __launch_bounds__(NT, D == 64 ? 2 : 3) void dkdv_kernel(BwdArgs a) {
  using T = Tile<D>;
  using WR = WaveRows<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BYTES + 2 * QL * 4 + (BIAS ? BIAS_WMAX * 4 : 0)];
  __shared__ __attribute__((aligned(16))) char krows_[4 * WR::BYTES];  // each wave's K rows
  __shared__ __attribute__((aligned(16))) char vrows_[4 * WR::BYTES];  // ... and V rows
  GDPA_LDS char* Qs = (GDPA_LDS char*)smem;
  GDPA_LDS char* dOs = Qs + T::BYTES;
  GDPA_LDS float* lse_s = (GDPA_LDS float*)(dOs + T::BYTES);
  GDPA_LDS float* D_s = lse_s + QL;
  GDPA_LDS float* bwin = D_s + QL;

  Item it;  // carries the sample's offsets and lengths
  if (!fetch_item(a.hdr, a.items_k, 1, it)) return;
  const int h = it.h, H = a.H, nb = a.nb;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int j0 = it.tile * KI;
  const int wkey = j0 + w * 32;
  const int jk = wkey + l32;
  const bool kvalid = jk < Lk;
  const bool wave_active = wkey < Lk;
  const int64_t krow = (int64_t)(kv0 + (kvalid ? jk : 0)) * H + h;

  // The wave's 32 K and V rows come in by direct loads (whole rows per instruction); they are
  // read as operands once the wave's loads have landed, below.
  GDPA_LDS char* kw_rows = (GDPA_LDS char*)krows_ + w * WR::BYTES;
  GDPA_LDS char* vw_rows = (GDPA_LDS char*)vrows_ + w * WR::BYTES;
  if (wave_active) {
    WR::issue(kw_rows, (const __bf16*)a.K, wkey, Lk, kv0, H, h, lane);
    WR::issue(vw_rows, (const __bf16*)a.V, wkey, Lk, kv0, H, h, lane);
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }
  // query tiles [qt0, nqt): from the causal start to the last tile whose window reaches the
  // item's last key
  const int nqt_all = (Lq + QL - 1) / QL;
  const int nqt = WIN ? win_end_qtile(min(Lk, j0 + KI) - 1, a.win, QL, nqt_all) : nqt_all;
  const int qt0 = CAUSAL ? j0 / QL : 0;
  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;
  // bias window in natural order (bwin[t] = bias[w_lo + t]), pre-multiplied by log2(e) for
  // softmax: a lane's 16 lookups are one base address plus constant offsets
  const float bmul = ACT == ACT_SOFTMAX ? LOG2E : 1.0f;
  int w_lo = 0;
  bool win_ok = false;

  TileLoader<D, NT> lq_, ldo_;
  float st_lse = 0.0f, st_d = 0.0f;
  auto load_q = [&](int qt) {
    lq_.load((const __bf16*)a.Q, qt * QL, Lq, a.q_shared ? 0 : q0, H, h, tid);
    ldo_.load((const __bf16*)a.dO, qt * QL, Lq, q0, H, h, tid);
    if (tid < QL) {
      const int i = qt * QL + tid;
      st_lse = 0.0f;
      st_d = 0.0f;
      if (ACT == ACT_SOFTMAX && i < Lq) {
        st_lse = a.lse[(int64_t)(q0 + i) * H + h] * LOG2E;
        st_d = a.Dvec[(int64_t)(q0 + i) * H + h];
      }
    }
  };
  if (qt0 < nqt && j0 < Lk) load_q(qt0);
  if (BIAS && qt0 < nqt && j0 < Lk) {  // staged while the first tile's loads are in flight
    // raw diagonals i - jk: i in [qt0 * QL, nqt * QL), jk in [j0, j0 + KI)
    w_lo = qt0 * QL - (j0 + KI - 1);
    win_ok = __builtin_amdgcn_readfirstlane((int)stage_bias_window(
                 bwin, bias_h, nb, w_lo, nqt * QL - 1 - j0, false, bmul, tid, NT)) != 0;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's K and V rows have landed
  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kop[s] = wave_active ? WR::op(kw_rows, s, lane) : zero_bf16x8();
    vop[s] = wave_active ? WR::op(vw_rows, s, lane) : zero_bf16x8();
  }
  for (int qt = qt0; qt < nqt && j0 < Lk; ++qt) {
    __syncthreads();
    lq_.store(Qs, tid);
    ldo_.store(dOs, tid);
    if (tid < QL) {
      lse_s[tid] = st_lse;
      D_s[tid] = st_d;
    }
    __syncthreads();
    if (qt + 1 < nqt) load_q(qt + 1);
    const int i0 = qt * QL;
    if (!wave_active) continue;
    if (CAUSAL && i0 + QL - 1 < wkey) continue;  // every query of the tile precedes every key
    if (WIN && i0 > min(wkey + 31, Lk - 1) + a.win - 1) continue;  // ... or is past every window
    const bool need_mask = (i0 + QL > Lq) || (wkey + 32 > Lk) || (CAUSAL && i0 < wkey + 31) ||
                           (WIN && i0 + QL - 1 > wkey + a.win - 1);
#pragma unroll  // unrolled: about 2 % faster than rolled, no spills
    for (int qb = 0; qb < 2; ++qb) {
      if (i0 + qb * 32 >= Lq) break;  // a half past the last query adds nothing (short queries)
      __builtin_amdgcn_sched_barrier(0);  // keep each 32-query block's loads inside its block
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(tile_row_op<D>(Qs, qb * 32, s, lane), kop[s], sacc);
        dpacc = mfma32(tile_row_op<D>(dOs, qb * 32, s, lane), vop[s], dpacc);
      }
      // scores in place: x = s * scale (* log2 e for softmax) + bias of diagonal i - jk, query
      // i = i0 + qb*32 + (r/4)*8 + 4g + r%4 for register r
      const float sc = ACT == ACT_SOFTMAX ? sl2 : a.scale;
      if (BIAS) {
        if (win_ok) {
          const GDPA_LDS float* bp = bwin + (i0 + qb * 32 + 4 * g - jk - w_lo);
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = sacc[r] * sc + bp[(r >> 2) * 8 + (r & 3)];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[r] = sacc[r] * sc +
                      bias_h[clampi(i0 + qb * 32 + (r >> 2) * 8 + 4 * g + (r & 3) - jk, 0, nb - 1)] * bmul;
        }
      } else {
        sacc *= sc;
      }
      // 8 queries at a time: probabilities and score gradients, then their two products
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        __builtin_amdgcn_sched_barrier(0);
        float pv[8], dsv[8];
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
          const int r4 = 2 * s2 + h4;
          const int ql = qb * 32 + r4 * 8 + 4 * g;
          const f32x4 l4 = *(const GDPA_LDS f32x4*)(lse_s + ql);
          const f32x4 d4 = *(const GDPA_LDS f32x4*)(D_s + ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            const int i = i0 + ql + e;
            float p;
            float ds = dscore<ACT>(sacc[r], sacc[r], l4[e], d4[e], dpacc[r], p);
            if (need_mask && (i >= Lq || !kvalid || (CAUSAL && jk > i) || (WIN && i > jk + a.win - 1))) {
              p = 0.0f;
              ds = 0.0f;
            }
            pv[4 * h4 + e] = p;
            dsv[4 * h4 + e] = ds;
          }
        }
        const bf16x8 pb = pack8(pv);
        const bf16x8 dsb = pack8(dsv);
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
          dv[n] = mfma32(tile_tr_op<D>(dOs, qb * 32 + 16 * s2, n, lane), pb, dv[n]);
          dk[n] = mfma32(tile_tr_op<D>(Qs, qb * 32 + 16 * s2, n, lane), dsb, dk[n]);
        }
      }
    }
  }
  if (!kvalid) return;
  __bf16* dkrow = (__bf16*)a.dK + krow * D;
  __bf16* dvrow = (__bf16*)a.dV + krow * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    store_acc_row_bf16(dkrow, dk[n], n, g, a.scale);
    store_acc_row_bf16(dvrow, dv[n], n, g, 1.0f);
  }
}

template <int D, int ACT, bool C, bool BI, bool WIN = false>
hipError_t launch_t(const BwdArgs& a, int gq, int gk, hipStream_t s) {
  if (gq > 0) {
    prof_before(PROF_DQ, s);
    hipLaunchKernelGGL((dq_kernel<D, ACT, C, BI, WIN>), dim3(gq), dim3(NT), 0, s, a);
    prof_after(PROF_DQ, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gk > 0) {
    prof_before(PROF_DKDV, s);
    hipLaunchKernelGGL((dkdv_kernel<D, ACT, C, BI, WIN>), dim3(gk), dim3(NT), 0, s, a);
    prof_after(PROF_DKDV, s);
  }
  return hipGetLastError();
}

template <int D, int ACT>
hipError_t launch_cb(const Prob& p, const BwdArgs& a, int gq, int gk, hipStream_t s) {
  const bool bias = p.nb > 0;
  if (p.win > 0)
    return bias ? launch_t<D, ACT, true, true, true>(a, gq, gk, s) : launch_t<D, ACT, true, false, true>(a, gq, gk, s);
  if (p.causal) return bias ? launch_t<D, ACT, true, true>(a, gq, gk, s) : launch_t<D, ACT, true, false>(a, gq, gk, s);
  return bias ? launch_t<D, ACT, false, true>(a, gq, gk, s) : launch_t<D, ACT, false, false>(a, gq, gk, s);
}

template <int D>
hipError_t launch_d(const Prob& p, const BwdArgs& a, int gq, int gk, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_cb<D, ACT_SOFTMAX>(p, a, gq, gk, s);
    case ACT_GELU_TANH: return launch_cb<D, ACT_GELU_TANH>(p, a, gq, gk, s);
    default: return launch_cb<D, ACT_SILU>(p, a, gq, gk, s);
  }
}

// D = 128: the direct-load kernels of gdpa_bwd_dl.h.
hipError_t launch_d128(const Prob& p, const BwdArgs& a, int gq, int gk, hipStream_t s) {
  if (gq > 0) {
    const hipError_t e = bwddl::launch_dq(p, a, persistent_grid(gq, 1), s);
    if (e != hipSuccess) return e;
  }
  return gk > 0 ? bwddl::launch_dkdv(p, a, persistent_grid(gk, 1), s) : hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const Prob& p, const BwdArgs& a, int grid_q, int grid_k, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_d<32>(p, a, grid_q, grid_k, s);
    case 64: return launch_d<64>(p, a, grid_q, grid_k, s);
    default: return launch_d128(p, a, grid_q, grid_k, s);
  }
}

}  // namespace gdpa
