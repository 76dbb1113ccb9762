// Backward kernels for D = 128 bf16 with direct global -> LDS tile loads and a two-stage LDS ring.
//
// Same method, work split and operand orientation as the register-staged kernels in
// gdpa_bwd_bf16.hip (recomputed scores, dQ and dK/dV in separate kernels with no atomics; page
// "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", JFA,
// GDPA and block-attention paragraphs). What differs:
//   * the streamed tiles (K and V for dQ, Q and dO for dK/dV) come in by direct loads (layout in
//     gdpa_dl.h) into one stage while the other stage is computed: no staging registers;
//   * each 64-row tile is processed in two 32-row halves, and the operands of a half are read
//     from LDS before its products are issued, so the products do not wait on one read each;
//   * the bias and the scale seed the score accumulators (acc = b / scale + q.k, then
//     x = acc * scale (* log2 e)), and masking runs only on tiles that reach a boundary.
#pragma once

#include <math.h>

#include "gdpa_common.h"
#include "gdpa_dl.h"
#include "gdpa_internal.h"
#include "gdpa_split.h"
#include "gdpa_tiles.h"  // store_acc_row_bf16

namespace gdpa {
namespace bwddl {

using namespace dl;

constexpr int NT = 256;         // threads per workgroup (4 waves)
constexpr int QI = BWD_Q_ITEM;  // queries per dQ item
constexpr int KL = BWD_K_LOOP;  // keys per tile in the dQ loop
constexpr int KI = BWD_K_ITEM;  // keys per dK/dV item
constexpr int QL = BWD_Q_LOOP;  // queries per tile in the dK/dV loop
static_assert(QI == 128 && KI == 128 && KL == ROWS && QL == ROWS, "kernels assume these tiles");
// A wave's skewed dS buffer: 128 columns of 32 rows, column-major with DSC floats per column
// (a multiple of 4 so that a column is read 16 bytes at a time, and 36 so that the 16 lanes of
// such a read start on distinct 4-bank groups).
constexpr int DSC = 36;
constexpr int DS_WAVE = 128 * DSC;

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Ties a value to its place in the instruction stream: the computation of x stays before this
// point (an empty volatile asm is ordered with the scheduling barriers around it).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

template <int ACT>
__device__ __forceinline__ float dscore(float x, float lse2, float Di, float dp, float& p) {
  // x: score in log2 units (softmax) or natural units (GDPA)
  if (ACT == ACT_SOFTMAX) {
    p = fast_exp2(x - lse2);
    return p * (dp - Di);
  }
  float y, dy;
  act_fwd_bwd(ACT, x, y, dy);
  p = y;
  return dp * dy;
}

// ------------------------------------------------------------------------------------------
// dQ: item = 128 queries of one (sample, head), 4 waves x 32 queries; loop over 64-key tiles.
// S^T = K Q^T and dP^T = V dO^T with lane = query, dQ^T += K^T dS^T with K^T read transposed.
// Bias gradient: the paired-diagonal sums of gdpa_bwd_bf16.hip over the wave's 32 x 64 block of
// dS, staged in a per-wave LDS buffer; every partial-row entry is written once.
// WIN: causal sliding window of a.win keys (query i sees keys i - win + 1 .. i).
template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
__global__ __launch_bounds__(NT, 1) void dq_dl_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char sk0_[TILE];
  __shared__ __attribute__((aligned(16))) char sv0_[TILE];
  __shared__ __attribute__((aligned(16))) char sk1_[TILE];
  __shared__ __attribute__((aligned(16))) char sv1_[TILE];
  __shared__ __attribute__((aligned(16))) float bwin_[BIAS ? BIAS_WMAX : 1];
  // bias-gradient buffer; at the start of an item, also where its dO and O rows land
  __shared__ __attribute__((aligned(16))) float dsbuf_[4 * DS_WAVE];
  __shared__ __attribute__((aligned(16))) char sink_[4 * 1024];  // prefetch loads land here
  __shared__ int flag_, next_[2];
  GDPA_LDS char* sk0 = (GDPA_LDS char*)sk0_;
  GDPA_LDS char* sv0 = (GDPA_LDS char*)sv0_;
  GDPA_LDS char* sk1 = (GDPA_LDS char*)sk1_;
  GDPA_LDS char* sv1 = (GDPA_LDS char*)sv1_;
  GDPA_LDS float* bwin = (GDPA_LDS float*)bwin_;
  GDPA_LDS int* nxt = (GDPA_LDS int*)next_;

  // Persistent: the workgroup works through its die's items (see ItemQueue). Each item claims
  // the next one as it starts, so the next record is at hand before the item ends. A short item
  // (one or two key tiles) also claims the item after the next, so that the next record is there
  // a whole item ahead and the next item's query rows can be prefetched during the short item's
  // last tile. (Claiming that far ahead on long items would hold back items that another
  // workgroup of the die could start sooner; prefetching at the end of a long item measured
  // slower, with more traffic, than leaving the next item's rows to its own loads.)
  ItemQueue qu;
  if (!queue_open(a.hdr, a.items_q, 0, qu)) return;
  {
    const int c0 = queue_claim(qu);
    if (threadIdx.x == 0) nxt[0] = c0;
    __syncthreads();
  }
  int idx = __builtin_amdgcn_readfirstlane(nxt[0]), nidx = qu.n;
  int rec = queue_fetch(qu, idx), rec1 = 0;
  bool have1 = false;  // nidx / rec1 hold the claimed next item
  for (;;) {
  if (idx >= qu.n) {  // this die's items are all claimed: take another die's
    idx = queue_steal(qu, nxt);
    if (idx >= qu.n) break;
    rec = queue_fetch(qu, idx);
    have1 = false;
  }
  const Item it = queue_record(rec);  // carries the sample's offsets and lengths
  int n2idx = qu.n, rec2 = 0;
  bool fetched = false;
  const int b = it.b, h = it.h, H = a.H, nb = a.nb;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i0 = it.tile * QI;
  const int wrow = i0 + w * 32;
  const int iq = wrow + l32;
  const bool qv = iq < Lq;
  const bool wave_active = wrow < Lq;
  const int64_t row = (int64_t)(q0 + (qv ? iq : 0)) * H + h;  // O, dO, lse, D row

  int nkt = (Lk + KL - 1) / KL;
  if (CAUSAL) nkt = min(nkt, (min(Lq, i0 + QI) - 1) / KL + 1);
  if (i0 >= Lq) nkt = 0;
  // key tiles of this item: all of them, or one chunk of a split tile, counted from the first
  // tile the item's sliding window reaches
  const int kt_first = WIN ? win_first_ktile(i0, a.win, KL) : 0;
  const int kt_lo = kt_first + it.lo, kt_hi = min(kt_first + it.hi, nkt);
  const bool short_item = kt_hi - kt_lo <= 2;

  // The item's query rows come in as direct-load tiles (whole cache lines per instruction) into
  // buffers idle until its first key tile: Q into stage 1, dO and O into the bias-gradient
  // buffer. Rows i0 .. i0 + 63 form the first tile of each, rows i0 + 64 .. i0 + 127 the second.
  const __bf16* Q = (const __bf16*)a.Q;
  const __bf16* dO = (const __bf16*)a.dO;
  GDPA_LDS char* rows_do = (GDPA_LDS char*)dsbuf_;
  GDPA_LDS char* rows_o = rows_do + 2 * TILE;
  const bool two = Lq > i0 + ROWS;  // the item has rows in its second 64
  {
    const int qbase = a.q_shared ? 0 : q0;
    issue_tile(sk1, Q, i0, Lq, qbase, H, h, w, lane);
    issue_tile(rows_do, dO, i0, Lq, q0, H, h, w, lane);
    if (ACT == ACT_SOFTMAX) issue_tile(rows_o, (const __bf16*)a.O, i0, Lq, q0, H, h, w, lane);
    if (two) {
      issue_tile(sv1, Q, i0 + ROWS, Lq, qbase, H, h, w, lane);
      issue_tile(rows_do + TILE, dO, i0 + ROWS, Lq, q0, H, h, w, lane);
      if (ACT == ACT_SOFTMAX) issue_tile(rows_o + TILE, (const __bf16*)a.O, i0 + ROWS, Lq, q0, H, h, w, lane);
    }
  }
  const float lse_row = ACT == ACT_SOFTMAX && qv ? a.lse[row] : 0.0f;
  // The bias window (raw diagonals iq - j: iq in [i0, i0 + QI), j in the item's tiles) comes in
  // the same way, bwin[t] = bias[clamp(w_hi - t)], and is scaled by 1 / scale after the wait.
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;
  int w_hi = 0, wcnt = 0;
  if (BIAS && kt_lo < kt_hi) {
    w_hi = i0 + QI - 1 - kt_lo * KL;
    wcnt = w_hi - (i0 - (kt_hi * KL - 1)) + 1;
    if (wcnt > BIAS_WMAX) wcnt = 0;  // too wide to stage: looked up in the table instead
    issue_window(bwin, bias_h, nb, w_hi, -1, wcnt, w, lane);
  }
  const bool win_ok = wcnt > 0;

  const int claim_a = have1 ? -1 : queue_claim(qu);       // the next item
  const int claim_b = short_item ? queue_claim(qu) : -1;  // the one after it
  const __bf16* K = (const __bf16*)a.K;
  const __bf16* V = (const __bf16*)a.V;
  if (kt_lo < kt_hi) {
    issue_tile(sk0, K, kt_lo * KL, Lk, kv0, H, h, w, lane);
    issue_tile(sv0, V, kt_lo * KL, Lk, kv0, H, h, w, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's row and window loads have landed
  __syncthreads();                // ... and everyone else's
  // wave w's 32 rows: tile w / 2, rows 32 (w % 2) ..; a wave past the item's rows uses zeros
  bf16x8 qop[D / 16], doop[D / 16];
  float part_d = 0.0f;
  {
    const int t = (w >> 1) * TILE, rb = (w & 1) * 32;
    const GDPA_LDS char* tq = (w >> 1) ? sv1 : sk1;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qop[s] = wave_active ? row_op(tq, rb, s, lane) : zero_bf16x8();
      doop[s] = wave_active ? row_op(rows_do + t, rb, s, lane) : zero_bf16x8();
      if (ACT == ACT_SOFTMAX && wave_active) {
        const bf16x8 ov = row_op(rows_o + t, rb, s, lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) part_d += (float)doop[s][e] * (float)ov[e];
      }
    }
  }
  float Di = 0.0f, lse2 = 0.0f;
  if (ACT == ACT_SOFTMAX) {
    Di = half_sum(part_d);
    if (qv) {
      lse2 = lse_row * LOG2E;
      // every chunk computes it; the first writes it
      if (g == 0 && split::chunk_index(it.chunk) == 0) a.Dvec[row] = Di;
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) dq[n] = f32x16{};

  const float sc = ACT == ACT_SOFTMAX ? a.scale * LOG2E : a.scale;
  const float inv_scale = 1.0f / a.scale;
  if (win_ok)  // read at the first key tile, after its barrier
    for (int t = tid; t < wcnt; t += NT) bwin[t] *= inv_scale;
  GDPA_LDS float* dsbuf = (GDPA_LDS float*)dsbuf_ + w * DS_WAVE;
  // Bias gradient: diagonal sums of each tile's 32 x 64 dS block. The block is stored skewed:
  // entry (row s, key j) in column j - s + 64, so a diagonal (fixed j - s) is one column, and the
  // columns a tile does not write stay zero. Lane t reads column 127 - t (diagonal t - 63: rows
  // 0..t, zeros below) and column 63 - t (diagonal t + 1: rows t + 1..31, zeros above); for
  // t >= 31 the first is the full diagonal t - 63 and the second is all zeros. Columns are
  // contiguous, so each lane reads its two columns with 8 + 8 16-byte loads, and the two sums
  // need no selects. A tile's sums are taken during the next tile's score products (or after the
  // loop), so the reads overlap matrix work and the partial-row store is not waited for at once.
  const GDPA_LDS float* cola = dsbuf + (127 - lane) * DSC;
  const GDPA_LDS float* colb = dsbuf + (63 - lane) * DSC;
  // row l32, key 4g in column 4g - l32 + 64; key 4g + o is o columns further
  GDPA_LDS float* dswr = dsbuf + (64 + 4 * g) * DSC - (DSC - 1) * l32;
  // (cleared at the first key tile, once every wave has read its rows from the buffer)
  auto clear_dsbuf = [&]() {  // each store covers 1 KiB of the buffer: 64 lanes on distinct banks
#pragma unroll
    for (int u = 0; u < DS_WAVE / 256; ++u)
      *(GDPA_LDS f32x4*)(dsbuf + 256 * u + 4 * lane) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  float carry = 0.0f;  // lanes t < 31: partial sum of diagonal t - 63 of the previous tile
  // partial row of this row block: canonical, or the chunk's slot row for a split tile
  float* part = !BIAS ? nullptr
                : it.slot < 0 ? a.dbias_part + ((int64_t)h * a.part_rows + it.aux * (QI / 32) + w) * nb
                              : a.dbias_part_x + ((int64_t)it.slot * (QI / 32) + w) * nb;
  float e_lo = 0.0f, e_hi = 0.0f;
  bool has_lo = false, has_hi = false;
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
  // the diagonals completed by the tile at key offset kp (s_a, s_b: its two column sums); pend =
  // a tile of this wave has been reduced
  auto finish = [&](int kp, float s_a, float s_b, bool pend) {
    // lanes t < 31 emit d = t + 1 (with the carried part), the others emit d = lane - 63;
    // absolute diagonal = wrow - kp + d
    float v;
    int dabs;
    if (lane < 31) {
      v = carry + s_b;
      carry = s_a;
      dabs = wrow - kp + lane + 1;
    } else {
      v = s_a;
      dabs = wrow - kp + lane - 63;
    }
    emit(dabs, v, pend);
  };
  auto col_sums = [&](float& s_a, float& s_b) {
    f32x4 va[8], vb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      va[k] = *(const GDPA_LDS f32x4*)(cola + 4 * k);
      vb[k] = *(const GDPA_LDS f32x4*)(colb + 4 * k);
    }
    s_a = 0.0f;
    s_b = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      s_a += va[e >> 2][e & 3];
      s_b += vb[e >> 2][e & 3];
    }
  };
  int k0_last = -1;

  // score accumulators of half kb of the tile at key offset k0, seeded with the bias / scale
  auto seed = [&](f32x16& sacc, int k0, int kb) {
    if (BIAS && win_ok) {
      const GDPA_LDS float* bp = bwin + (w_hi - iq + k0 + kb * 32 + 4 * g);
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = bp[(r >> 2) * 8 + (r & 3)];
    } else if (BIAS) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[r] = bias_h[clampi(iq - (k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3)), 0, nb - 1)] * inv_scale;
    } else {
      sacc = f32x16{};
    }
  };

  // One key tile in four sections, each a run of matrix products with independent vector work
  // laid between them (a wave issues in order, so work placed between products runs while they
  // execute):
  //   A  scores S^T, dP^T of keys 0..31, with the previous tile's column sums (bias) and the
  //      transposed K^T operands of keys 0..31;
  //   B  scores of keys 32..63, with the gradient dS^T of keys 0..31 and the K^T operands of
  //      keys 32..63;
  //   C  dQ^T += K^T dS^T for keys 0..31, with the gradient of keys 32..63;
  //   D  dQ^T += K^T dS^T for keys 32..63.
  // MASK: the tile reaches the end of the keys, the causal diagonal or the end of the queries.
  auto tile = [&](auto mask_c, const GDPA_LDS char* __restrict__ Ks, const GDPA_LDS char* __restrict__ Vs, int k0) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int kp = k0_last;
    k0_last = k0;
    int lim[2], lo[2];  // key offset o of register r (8 (r / 4) + r % 4) valid for lo <= o < lim
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int l = Lk - (k0 + kb * 32);
      if (CAUSAL) l = min(l, iq - (k0 + kb * 32) + 1);
      lim[kb] = qv ? l - 4 * g : -64;
      lo[kb] = WIN ? iq - a.win + 1 - (k0 + kb * 32) - 4 * g : -64;
    }
    // gradient of element r of half kb (register r holds key kb*32 + 8(r/4) + 4g + r%4)
    auto grad = [&](int kb, int r, float sv, float dpv) {
      float p;
      float v = dscore<ACT>(sv * sc, lse2, Di, dpv, p);
      if (MASK && ((r >> 2) * 8 + (r & 3) >= lim[kb] || (WIN && (r >> 2) * 8 + (r & 3) < lo[kb]))) v = 0.0f;
      return v;
    };
    f32x16 sacc0, sacc1, dpacc0 = f32x16{}, dpacc1 = f32x16{};
    seed(sacc0, k0, 0);
    bf16x8 kr[D / 16], vr[D / 16], kr1[D / 16], vr1[D / 16];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kr[s] = row_op(Ks, 0, s, lane);
      vr[s] = row_op(Vs, 0, s, lane);
    }
    bf16x8 kt0[D / 32], kt1[D / 32], ku0[D / 32], ku1[D / 32];
    f32x2 sab = {0.0f, 0.0f};  // the two column sums advance together
    f32x4 va[8], vb[8];
    __builtin_amdgcn_sched_barrier(0);
    // A: per pair of products, the operands two steps ahead, the column reads of four rows, one
    // transposed operand, and the sums of the rows read two steps earlier
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 2 < D / 16) {
        kr[s + 2] = row_op(Ks, 0, s + 2, lane);
        vr[s + 2] = row_op(Vs, 0, s + 2, lane);
      } else {
        kr1[s - 6] = row_op(Ks, 32, s - 6, lane);
        vr1[s - 6] = row_op(Vs, 32, s - 6, lane);
      }
      sacc0 = mfma32(kr[s], qop[s], sacc0);
      dpacc0 = mfma32(vr[s], doop[s], dpacc0);
      if (BIAS) {
        va[s] = *(const GDPA_LDS f32x4*)(cola + 4 * s);
        vb[s] = *(const GDPA_LDS f32x4*)(colb + 4 * s);
        if (s >= 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sab += f32x2{va[s - 2][e], vb[s - 2][e]};
        }
      }
      if (s & 1) kt1[s >> 1] = tr_op(Ks, 16, s >> 1, lane);
      else kt0[s >> 1] = tr_op(Ks, 0, s >> 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (BIAS) {
#pragma unroll
      for (int e = 24; e < 32; ++e) sab += f32x2{va[e >> 2][e & 3], vb[e >> 2][e & 3]};
      finish(kp, sab[0], sab[1], kp >= 0);
    }
    seed(sacc1, k0, 1);  // (read here rather than with the first seed: measured faster)
    __builtin_amdgcn_sched_barrier(0);
    // B: per pair of products, the operands two steps ahead, the gradient of two elements of
    // half 0 and one transposed operand of half 1
    float ds0[16], ds1[16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 2 < D / 16) {
        kr1[s + 2] = row_op(Ks, 32, s + 2, lane);
        vr1[s + 2] = row_op(Vs, 32, s + 2, lane);
      }
      sacc1 = mfma32(kr1[s], qop[s], sacc1);
      dpacc1 = mfma32(vr1[s], doop[s], dpacc1);
      ds0[2 * s] = grad(0, 2 * s, sacc0[2 * s], dpacc0[2 * s]);
      ds0[2 * s + 1] = grad(0, 2 * s + 1, sacc0[2 * s + 1], dpacc0[2 * s + 1]);
      pin(ds0[2 * s]);
      pin(ds0[2 * s + 1]);
      if (s & 1) ku1[s >> 1] = tr_op(Ks, 48, s >> 1, lane);
      else ku0[s >> 1] = tr_op(Ks, 32, s >> 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (BIAS) {  // the column reads of section A are done before the buffer is rewritten
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int r = 0; r < 16; ++r) dswr[((r >> 2) * 8 + (r & 3)) * DSC] = ds0[r];
    }
    const bf16x8 d00 = pack8(&ds0[0]), d01 = pack8(&ds0[8]);
    __builtin_amdgcn_sched_barrier(0);
    // C: per pair of products, the gradient of four elements of half 1
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      dq[n] = mfma32(kt0[n], d00, dq[n]);
      dq[n] = mfma32(kt1[n], d01, dq[n]);
#pragma unroll
      for (int r = 4 * n; r < 4 * n + 4; ++r) {
        ds1[r] = grad(1, r, sacc1[r], dpacc1[r]);
        pin(ds1[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (BIAS) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dswr[(32 + (r >> 2) * 8 + (r & 3)) * DSC] = ds1[r];
    }
    const bf16x8 d10 = pack8(&ds1[0]), d11 = pack8(&ds1[8]);
    __builtin_amdgcn_sched_barrier(0);
    // D
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      dq[n] = mfma32(ku0[n], d10, dq[n]);
      dq[n] = mfma32(ku1[n], d11, dq[n]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run_tile = [&](const GDPA_LDS char* __restrict__ Ks, const GDPA_LDS char* __restrict__ Vs, int k0) {
    const bool need_mask = __builtin_amdgcn_readfirstlane(
        (int)((k0 + KL > Lk) || (CAUSAL && k0 + KL - 1 > wrow) || (wrow + 32 > Lq) ||
              (WIN && k0 < wrow + 32 - a.win))) != 0;
    if (need_mask) tile(BoolC<true>{}, Ks, Vs, k0);
    else tile(BoolC<false>{}, Ks, Vs, k0);
  };

  // whether this wave computes key tile kt: not wholly after its last query (causal) nor wholly
  // before its first query's window (the bias-gradient reduction assumes the same range)
  auto wave_needs = [&](int kt) {
    return wave_active && !(CAUSAL && kt * KL > wrow + 31) && !(WIN && (kt + 1) * KL <= wrow - a.win + 1);
  };
  // Two stages, loop unrolled by two so each stage is a distinct LDS object: the direct loads
  // into one stage stay in flight while the other stage is read.
  // At the start of tile kt (after its barrier): on the first tile, the records of the items
  // claimed by this one are fetched; on the last tile of a short item, the next item's query rows
  // are prefetched if its record is there (no later tile wait of this item covers those loads).
  GDPA_LDS char* sink = (GDPA_LDS char*)sink_ + w * 1024;
  const int kt_pf = kt_hi - 1;
  auto fetch_claimed = [&]() {
    if (!have1) {
      nidx = __builtin_amdgcn_readfirstlane(nxt[0]);
      rec1 = queue_fetch(qu, nidx);
    }
    if (short_item) {
      n2idx = __builtin_amdgcn_readfirstlane(nxt[1]);
      rec2 = queue_fetch(qu, n2idx);
    }
    fetched = true;
  };
  auto at_tile = [&](int kt) {
    if (kt == kt_lo) {
      fetch_claimed();
      if (BIAS) clear_dsbuf();
    }
    if (short_item && kt == kt_pf && (have1 || kt > kt_lo) && nidx < qu.n) {
      const Item nx = queue_record(rec1);
      const int r0 = nx.tile * QI + w * 32;
      prefetch_rows32<D>(sink, Q, r0, nx.lq, a.q_shared ? 0 : nx.q0, H, nx.h, lane);
      prefetch_rows32<D>(sink, dO, r0, nx.lq, nx.q0, H, nx.h, lane);
      if (ACT == ACT_SOFTMAX) prefetch_rows32<D>(sink, (const __bf16*)a.O, r0, nx.lq, nx.q0, H, nx.h, lane);
    }
  };
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads for tile kt have landed
    if (kt == kt_lo && tid == 0) {
      nxt[0] = claim_a;
      nxt[1] = claim_b;
    }
    __syncthreads();                // ... and everyone else's; tile kt - 1 is done with stage 1
    if (kt + 1 < kt_hi) {
      issue_tile(sk1, K, (kt + 1) * KL, Lk, kv0, H, h, w, lane);
      issue_tile(sv1, V, (kt + 1) * KL, Lk, kv0, H, h, w, lane);
    }
    at_tile(kt);
    if (wave_needs(kt)) run_tile(sk0, sv0, kt * KL);
    if (kt + 1 >= kt_hi) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 2 < kt_hi) {
      issue_tile(sk0, K, (kt + 2) * KL, Lk, kv0, H, h, w, lane);
      issue_tile(sv0, V, (kt + 2) * KL, Lk, kv0, H, h, w, lane);
    }
    at_tile(kt + 1);
    if (wave_needs(kt + 1)) run_tile(sk1, sv1, (kt + 1) * KL);
  }

  if (BIAS && k0_last >= 0) {
    // the sums of this wave's last tile, then its 31 carried diagonals d = t - 63
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float s_a, s_b;
    col_sums(s_a, s_b);
    finish(k0_last, s_a, s_b, true);
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
  if (it.slot >= 0) {
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
      split::combine_dq_tile(a, b, it.tile, h, n, first);
  } else if (qv) {
    if (a.dq_f32) {  // shared Q: this sample's gradient, summed over samples afterwards
#pragma unroll
      for (int n = 0; n < D / 32; ++n) store_acc_row_f32(a.dq_f32 + row * D, dq[n], n, g, a.scale);
    } else {
      __bf16* dqrow = (__bf16*)a.dQ + row * D;
#pragma unroll
      for (int n = 0; n < D / 32; ++n) store_acc_row_bf16(dqrow, dq[n], n, g, a.scale);
    }
  }
  if (!fetched) {  // an item without key tiles: publish the claims now
    if (tid == 0) {
      nxt[0] = claim_a;
      nxt[1] = claim_b;
    }
    __syncthreads();
    fetch_claimed();
  }
  __syncthreads();  // this item's LDS (stages, bias window, flags) is free again
  idx = nidx;
  rec = rec1;
  have1 = short_item;
  nidx = n2idx;
  rec1 = rec2;
  }
}

// ------------------------------------------------------------------------------------------
// dK, dV: item = 128 keys of one (sample, head), 4 waves x 32 keys; loop over 64-query tiles.
// S = Q K^T and dP = dO V^T with lane = key; dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
// read transposed from the query tiles. The softmax row terms (lse, D) of a query tile come in
// by 4-byte direct loads beside the tile itself.
// WIN: causal sliding window of a.win keys (key j is seen by queries j .. j + win - 1).
template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
__global__ __launch_bounds__(NT, 1) void dkdv_dl_kernel(BwdArgs a) {
  constexpr bool SM = ACT == ACT_SOFTMAX;
  __shared__ __attribute__((aligned(16))) char sq0_[TILE];
  __shared__ __attribute__((aligned(16))) char so0_[TILE];
  __shared__ __attribute__((aligned(16))) char sq1_[TILE];
  __shared__ __attribute__((aligned(16))) char so1_[TILE];
  __shared__ __attribute__((aligned(16))) float rt_[SM ? 2 * 2 * QL : 1];  // [stage][lse, D][QL]
  __shared__ __attribute__((aligned(16))) float bwin_[BIAS ? BIAS_WMAX : 1];
  __shared__ __attribute__((aligned(16))) char vrows_[2 * TILE];  // the item's V rows
  __shared__ __attribute__((aligned(16))) char sink_[4 * 1024];   // prefetch loads land here
  __shared__ int flag_, next_[2];
  GDPA_LDS char* sq0 = (GDPA_LDS char*)sq0_;
  GDPA_LDS char* so0 = (GDPA_LDS char*)so0_;
  GDPA_LDS char* sq1 = (GDPA_LDS char*)sq1_;
  GDPA_LDS char* so1 = (GDPA_LDS char*)so1_;
  GDPA_LDS float* rt = (GDPA_LDS float*)rt_;
  GDPA_LDS float* bwin = (GDPA_LDS float*)bwin_;
  GDPA_LDS int* nxt = (GDPA_LDS int*)next_;

  // Persistent, with the claims, record fetches and next-item prefetch of the dQ kernel.
  ItemQueue qu;
  if (!queue_open(a.hdr, a.items_k, 1, qu)) return;
  {
    const int c0 = queue_claim(qu);
    if (threadIdx.x == 0) nxt[0] = c0;
    __syncthreads();
  }
  int idx = __builtin_amdgcn_readfirstlane(nxt[0]), nidx = qu.n;
  int rec = queue_fetch(qu, idx), rec1 = 0;
  bool have1 = false;  // nidx / rec1 hold the claimed next item
  for (;;) {
  if (idx >= qu.n) {  // this die's items are all claimed: take another die's
    idx = queue_steal(qu, nxt);
    if (idx >= qu.n) break;
    rec = queue_fetch(qu, idx);
    have1 = false;
  }
  const Item it = queue_record(rec);  // carries the sample's offsets and lengths
  int n2idx = qu.n, rec2 = 0;
  bool fetched = false;
  const int b = it.b, h = it.h, H = a.H, nb = a.nb;
  const int q0 = it.q0, Lq = it.lq;
  const int kv0 = it.kv0, Lk = it.lk;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = it.tile * KI;
  const int wkey = j0 + w * 32;
  const int jk = wkey + l32;
  const bool kvalid = jk < Lk;
  const bool wave_active = wkey < Lk;
  const int64_t krow = (int64_t)(kv0 + (kvalid ? jk : 0)) * H + h;

  const int nqt = (Lq + QL - 1) / QL;
  const int qt0 = CAUSAL ? j0 / QL : 0;
  // one past the last query tile whose window reaches this key tile
  const int qend = WIN ? win_end_qtile(min(Lk, j0 + KI) - 1, a.win, QL, nqt) : nqt;
  const int nt = j0 < Lk && qt0 < qend ? qend - qt0 : 0;  // query tiles this key tile visits
  // the item's query tiles qt0 + [t_lo, t_hi): all of them, or one chunk of a split tile
  const int t_lo = it.lo, t_hi = min(it.hi, nt);
  const bool short_item = t_hi - t_lo <= 2;

  const __bf16* Q = (const __bf16*)a.Q;
  const __bf16* dO = (const __bf16*)a.dO;
  // Direct loads of query tile qt (Q, dO and, for softmax, its lse and D entries) into a stage.
  // Waves 0 and 1 fetch the 64 lse / D values (one 4-byte load per lane, rows past the end
  // repeat the tile's first row).
  auto issue = [&](GDPA_LDS char* sq, GDPA_LDS char* so, GDPA_LDS float* srt, int qt) {
    issue_tile(sq, Q, qt * QL, Lq, a.q_shared ? 0 : q0, H, h, w, lane);
    issue_tile(so, dO, qt * QL, Lq, q0, H, h, w, lane);
    if (SM && w < 2) {
      const int r0 = qt * QL, n = min(QL, Lq - r0);
      const float* src = (w == 0 ? a.lse : a.Dvec) + ((int64_t)(q0 + r0) * H + h);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, ((n - 1) * H + 1) * 4, 0x00020000);
      const int r = lane < n ? lane : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GDPA_LDS void*)(srt + w * QL), 4, r * H * 4, 0, 0, 0);
    }
  };
  // Query tiles are visited last to first: every key tile of a sample then starts at the same
  // query tile, so the key tiles of one (sample, head), which the scheduler starts together on
  // one die, stream the shared query tiles through its L2 in step.
  // The item's key rows come in as direct-load tiles (whole cache lines per instruction): K into
  // stage 1, idle until the first query tile, and V into their own buffer. Keys j0 .. j0 + 63
  // form the first tile of each, keys j0 + 64 .. j0 + 127 the second.
  const __bf16* K = (const __bf16*)a.K;
  const __bf16* V = (const __bf16*)a.V;
  GDPA_LDS char* vrows = (GDPA_LDS char*)vrows_;
  issue_tile(sq1, K, j0, Lk, kv0, H, h, w, lane);
  issue_tile(vrows, V, j0, Lk, kv0, H, h, w, lane);
  if (Lk > j0 + ROWS) {
    issue_tile(so1, K, j0 + ROWS, Lk, kv0, H, h, w, lane);
    issue_tile(vrows + TILE, V, j0 + ROWS, Lk, kv0, H, h, w, lane);
  }
  // The bias window in natural order (raw diagonals i - jk: i in the item's query tiles, jk in
  // [j0, j0 + KI)) comes in the same way, bwin[t] = bias[clamp(w_lo + t)], and is scaled by
  // 1 / scale after the wait: a lane's 16 lookups are then one base address plus constant offsets.
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;
  int w_lo = 0, wcnt = 0;
  if (BIAS && t_lo < t_hi) {
    w_lo = (qt0 + t_lo) * QL - (j0 + KI - 1);
    wcnt = (qt0 + t_hi) * QL - 1 - j0 - w_lo + 1;
    if (wcnt > BIAS_WMAX) wcnt = 0;  // too wide to stage: looked up in the table instead
    issue_window(bwin, bias_h, nb, w_lo, 1, wcnt, w, lane);
  }
  const bool win_ok = wcnt > 0;
  const int claim_a = have1 ? -1 : queue_claim(qu);       // the next item
  const int claim_b = short_item ? queue_claim(qu) : -1;  // the one after it
  if (t_lo < t_hi) issue(sq0, so0, rt, qt0 + t_hi - 1);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's row and window loads have landed
  __syncthreads();                // ... and everyone else's
  // wave w's 32 keys: tile w / 2, rows 32 (w % 2) ..; a wave past the item's keys uses zeros
  bf16x8 kop[D / 16], vop[D / 16];
  {
    const GDPA_LDS char* tk = (w >> 1) ? so1 : sq1;
    const GDPA_LDS char* tv = vrows + (w >> 1) * TILE;
    const int rb = (w & 1) * 32;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kop[s] = wave_active ? row_op(tk, rb, s, lane) : zero_bf16x8();
      vop[s] = wave_active ? row_op(tv, rb, s, lane) : zero_bf16x8();
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }
  const float sc = SM ? a.scale * LOG2E : a.scale;
  const float inv_scale = 1.0f / a.scale;
  if (win_ok)  // read at the first query tile, after its barrier
    for (int t = tid; t < wcnt; t += NT) bwin[t] *= inv_scale;

  auto tile = [&](const GDPA_LDS char* __restrict__ Qs, const GDPA_LDS char* __restrict__ dOs,
                  const GDPA_LDS float* srt, int i0) {
    const bool need_mask = __builtin_amdgcn_readfirstlane(
        (int)((i0 + QL > Lq) || (wkey + 32 > Lk) || (CAUSAL && i0 < wkey + 31) ||
              (WIN && i0 + QL - 1 > wkey + a.win - 1))) != 0;
    auto half = [&](int qb) {
      const int ib = i0 + qb * 32 + 4 * g;  // query of register r: ib + (r / 4) * 8 + r % 4
      f32x16 sacc, dpacc = f32x16{};
      if (BIAS && win_ok) {
        const GDPA_LDS float* bp = bwin + (ib - jk - w_lo);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = bp[(r >> 2) * 8 + (r & 3)];
      } else if (BIAS) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = bias_h[clampi(ib + (r >> 2) * 8 + (r & 3) - jk, 0, nb - 1)] * inv_scale;
      } else {
        sacc = f32x16{};
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 qr[D / 16], dr[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        qr[s] = row_op(Qs, qb * 32, s, lane);
        dr[s] = row_op(dOs, qb * 32, s, lane);
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(qr[s], kop[s], sacc);
        dpacc = mfma32(dr[s], vop[s], dpacc);
      }
      // the transposed dO^T operands of this half's dV products, read now so they arrive during
      // the gradient arithmetic
      bf16x8 ot[2][D / 32];
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        ot[0][n] = tr_op(dOs, qb * 32, n, lane);
        ot[1][n] = tr_op(dOs, qb * 32 + 16, n, lane);
      }
      // the 16 operand reads, then the 16 products each followed by one transposed read
#pragma unroll
      for (int i = 0; i < D / 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);

      float pv[16], dsv[16];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 l4 = {}, d4 = {};
        if (SM) {
          l4 = *(const GDPA_LDS f32x4*)(srt + qb * 32 + m * 8 + 4 * g);
          d4 = *(const GDPA_LDS f32x4*)(srt + QL + qb * 32 + m * 8 + 4 * g);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          float p;
          dsv[r] = dscore<ACT>(sacc[r] * sc, l4[e] * LOG2E, d4[e], dpacc[r], p);
          pv[r] = p;
        }
      }
      if (need_mask) {
        int hi = kvalid ? Lq - ib : -64;    // query offsets at or past hi are invalid
        if (WIN) hi = min(hi, jk + a.win - ib);  // ... and those past the key's window
        const int lo = CAUSAL ? jk - ib : -64;  // query offsets below lo precede the key
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = (r >> 2) * 8 + (r & 3);
          if (off >= hi || off < lo) {
            pv[r] = 0.0f;
            dsv[r] = 0.0f;
          }
        }
      }
      const bf16x8 pb0 = pack8(&pv[0]), pb1 = pack8(&pv[8]);
      const bf16x8 db0 = pack8(&dsv[0]), db1 = pack8(&dsv[8]);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 qt[2][D / 32];
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        qt[0][n] = tr_op(Qs, qb * 32, n, lane);
        qt[1][n] = tr_op(Qs, qb * 32 + 16, n, lane);
      }
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        dv[n] = mfma32(ot[0][n], pb0, dv[n]);
        dv[n] = mfma32(ot[1][n], pb1, dv[n]);
      }
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        dk[n] = mfma32(qt[0][n], db0, dk[n]);
        dk[n] = mfma32(qt[1][n], db1, dk[n]);
      }
      // the dV products interleaved with the Q^T reads, then the dK products
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < D / 16; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // The two halves straight-line, with or without a bias (a loop over the halves copied the
    // dK/dV accumulators on its back edge: 6-10 % slower without a bias).
    half(0);
    half(1);
  };

  // whether this wave computes the query tile at i0: not wholly before its first key (causal)
  // nor wholly after the window of its last key
  auto wave_needs = [&](int i0) {
    return wave_active && !(CAUSAL && i0 + QL - 1 < wkey) && !(WIN && i0 > min(wkey + 31, Lk - 1) + a.win - 1);
  };
  // At the start of query tile t (after its barrier): on the first, the records of the items
  // claimed by this one are fetched; on the last tile of a short item, the next item's key rows
  // are prefetched if its record is there.
  GDPA_LDS char* sink = (GDPA_LDS char*)sink_ + w * 1024;
  auto fetch_claimed = [&]() {
    if (!have1) {
      nidx = __builtin_amdgcn_readfirstlane(nxt[0]);
      rec1 = queue_fetch(qu, nidx);
    }
    if (short_item) {
      n2idx = __builtin_amdgcn_readfirstlane(nxt[1]);
      rec2 = queue_fetch(qu, n2idx);
    }
    fetched = true;
  };
  auto at_tile = [&](int t) {
    if (t == t_hi - 1) fetch_claimed();
    if (short_item && t == t_lo && (have1 || t < t_hi - 1) && nidx < qu.n) {
      const Item nx = queue_record(rec1);
      const int r0 = nx.tile * KI + w * 32;
      prefetch_rows32<D>(sink, K, r0, nx.lk, nx.kv0, H, nx.h, lane);
      prefetch_rows32<D>(sink, V, r0, nx.lk, nx.kv0, H, nx.h, lane);
    }
  };
  // Two stages, as in the dQ kernel.
  GDPA_LDS float* rt0 = rt;
  GDPA_LDS float* rt1 = rt + (SM ? 2 * QL : 0);
  for (int t = t_hi - 1; t >= t_lo; t -= 2) {
    __builtin_amdgcn_s_waitcnt(0);
    if (t == t_hi - 1 && tid == 0) {
      nxt[0] = claim_a;
      nxt[1] = claim_b;
    }
    __syncthreads();
    if (t - 1 >= t_lo) issue(sq1, so1, rt1, qt0 + t - 1);
    at_tile(t);
    {
      const int i0 = (qt0 + t) * QL;
      if (wave_needs(i0)) tile(sq0, so0, rt0, i0);
    }
    if (t - 1 < t_lo) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t - 2 >= t_lo) issue(sq0, so0, rt0, qt0 + t - 2);
    at_tile(t - 1);
    {
      const int i0 = (qt0 + t - 1) * QL;
      if (wave_needs(i0)) tile(sq1, so1, rt1, i0);
    }
  }
  if (it.slot >= 0) {
    // chunk of a split tile: fp32 partial rows; the workgroup that completes the tile combines
    // its chunks in order
    if (wave_active) {
      const int64_t prow = ((int64_t)it.slot * KI + w * 32 + l32) * D;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          *(f32x4*)(a.part_dk + prow + n * 32 + r4 * 8 + 4 * g) =
              f32x4{dk[n][4 * r4], dk[n][4 * r4 + 1], dk[n][4 * r4 + 2], dk[n][4 * r4 + 3]};
          *(f32x4*)(a.part_dv + prow + n * 32 + r4 * 8 + 4 * g) =
              f32x4{dv[n][4 * r4], dv[n][4 * r4 + 1], dv[n][4 * r4 + 2], dv[n][4 * r4 + 3]};
        }
    }
    const int first = it.slot - split::chunk_index(it.chunk), n = split::chunk_count(it.chunk);
    if (split::chunk_done(a.split_cnt_k + first, n, (GDPA_LDS int*)&flag_))
      split::combine_dkdv_tile(a, b, it.tile, h, n, first);
  } else if (kvalid) {
    __bf16* dkrow = (__bf16*)a.dK + krow * D;
    __bf16* dvrow = (__bf16*)a.dV + krow * D;
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      store_acc_row_bf16(dkrow, dk[n], n, g, a.scale);
      store_acc_row_bf16(dvrow, dv[n], n, g, 1.0f);
    }
  }
  if (!fetched) {  // an item without query tiles: publish the claims now
    if (tid == 0) {
      nxt[0] = claim_a;
      nxt[1] = claim_b;
    }
    __syncthreads();
    fetch_claimed();
  }
  __syncthreads();  // this item's LDS (stages, rows, bias window, flags) is free again
  idx = nidx;
  rec = rec1;
  have1 = short_item;
  nidx = n2idx;
  rec1 = rec2;
  }
}

template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
hipError_t launch_dq_t(const BwdArgs& a, int grid, hipStream_t s) {
  prof_before(PROF_DQ, s);
  hipLaunchKernelGGL((dq_dl_kernel<ACT, CAUSAL, BIAS, WIN>), dim3(grid), dim3(NT), 0, s, a);
  prof_after(PROF_DQ, s);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_dq_cb(const Prob& p, const BwdArgs& a, int grid, hipStream_t s) {
  const bool bias = p.nb > 0;
  if (p.win > 0) return bias ? launch_dq_t<ACT, true, true, true>(a, grid, s) : launch_dq_t<ACT, true, false, true>(a, grid, s);
  if (p.causal) return bias ? launch_dq_t<ACT, true, true>(a, grid, s) : launch_dq_t<ACT, true, false>(a, grid, s);
  return bias ? launch_dq_t<ACT, false, true>(a, grid, s) : launch_dq_t<ACT, false, false>(a, grid, s);
}

template <int ACT, bool CAUSAL, bool BIAS, bool WIN = false>
hipError_t launch_dkdv_t(const BwdArgs& a, int grid, hipStream_t s) {
  prof_before(PROF_DKDV, s);
  hipLaunchKernelGGL((dkdv_dl_kernel<ACT, CAUSAL, BIAS, WIN>), dim3(grid), dim3(NT), 0, s, a);
  prof_after(PROF_DKDV, s);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_dkdv_cb(const Prob& p, const BwdArgs& a, int grid, hipStream_t s) {
  const bool bias = p.nb > 0;
  if (p.win > 0) return bias ? launch_dkdv_t<ACT, true, true, true>(a, grid, s) : launch_dkdv_t<ACT, true, false, true>(a, grid, s);
  if (p.causal) return bias ? launch_dkdv_t<ACT, true, true>(a, grid, s) : launch_dkdv_t<ACT, true, false>(a, grid, s);
  return bias ? launch_dkdv_t<ACT, false, true>(a, grid, s) : launch_dkdv_t<ACT, false, false>(a, grid, s);
}

inline hipError_t launch_dkdv(const Prob& p, const BwdArgs& a, int grid, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_dkdv_cb<ACT_SOFTMAX>(p, a, grid, s);
    case ACT_GELU_TANH: return launch_dkdv_cb<ACT_GELU_TANH>(p, a, grid, s);
    default: return launch_dkdv_cb<ACT_SILU>(p, a, grid, s);
  }
}

inline hipError_t launch_dq(const Prob& p, const BwdArgs& a, int grid, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_dq_cb<ACT_SOFTMAX>(p, a, grid, s);
    case ACT_GELU_TANH: return launch_dq_cb<ACT_GELU_TANH>(p, a, grid, s);
    default: return launch_dq_cb<ACT_SILU>(p, a, grid, s);
  }
}

}  // namespace bwddl
}  // namespace gdpa
