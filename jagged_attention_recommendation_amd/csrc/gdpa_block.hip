// Block-aligned attention with rotary position embeddings, D = 128 bf16.
//
// Page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model",
// block-attention paragraph: the sequence is cut into fixed blocks of 64 tokens and each block
// attends only within itself, so a whole block's scores fit one tile. The kernels here use that:
// no online softmax correction (the row maximum and sum are taken over the one tile), no
// logsumexp written to or read from HBM, and no separate pass for the backward's row term
// D_i = sum_j p_ij dp_ij (formed in the tile from P and dP). The rotary embedding is applied to
// Q and K in the prologue, and its backward (the rotation turned back) runs in the epilogue on
// the fp32 gradients.
//
// Work item: one (sample, 64-token block, head) from the jagged scheduler (query tiles of 64
// rows). Tiles come in by direct loads (layout in gdpa_dl.h), rows past the sample's end repeat
// its first row and are masked. Rotation: the pair (2m, 2m+1) of a row at position p (counted
// from the sample's first token) turns by p * base^(-2m/D) radians; the angle's fractional
// revolutions are formed in fp64 and the sine and cosine taken by the hardware in revolutions.
//   forward  (2 waves, lane = query): S^T = K_r Q_r^T, P in the tile, O^T = V^T P^T. The rotated
//            operands enter the score product as bf16 hi + lo parts (see rope_tiles).
//   backward (4 waves): waves 0-1, lane = query: S^T, dP^T = V dO^T, P, D_i, dS^T and
//            dQ_r^T = K_r^T dS^T; they leave each row's log2-sum-exp and D_i in LDS. Waves 2-3,
//            lane = key: S = Q_r K_r^T, dP = dO V^T, P and dS from those row terms,
//            dV^T = dO^T P, dK_r^T = Q_r^T dS. dQ and dK are rotated back in fp32. With the
//            rotation, every product that takes a rotated operand takes its hi and lo parts.
#include <math.h>

#include "gdpa_common.h"
#include "gdpa_dl.h"
#include "gdpa_internal.h"
#include "gdpa_tiles.h"  // store_acc_row_bf16

namespace gdpa {
namespace blk {

using namespace dl;

constexpr int BL = BLOCK_TOKENS;
static_assert(BL == ROWS, "a block is one direct-load tile");
constexpr double INV_2PI = 0.15915494309189533577;

// Revolutions per position of pair m: base^(-2m/D) / (2 pi), for m = 0 .. D/2 - 1, into LDS.
__device__ __forceinline__ void rope_table(GDPA_LDS double* c, double log2_base, int tid) {
  if (tid < D / 2) c[tid] = exp2(-(2.0 * tid / D) * log2_base) * INV_2PI;
}

// Sine and cosine of the angle of a pair at position pos: frac(pos * c) revolutions. pos * c
// reaches ~2.6e3 revolutions at position 16384, where an fp32 product would keep only ~13 bits
// of the fraction; in fp64 the fraction is exact to ~1e-12.
__device__ __forceinline__ void rope_sc(double c, int pos, float& sn, float& cs) {
  const double rev = (double)pos * c;
  const float f = (float)(rev - floor(rev));
  sn = __builtin_amdgcn_sinf(f);
  cs = __builtin_amdgcn_cosf(f);
}

// Rotate rows [0, n) of the Q and K tiles in place. The rotated value x (fp32) is kept as two
// bf16 parts, hi = bf16(x) in the tile and lo = bf16(x - hi) in a second tile, so the score
// product can be formed as hi.hi + lo.hi + hi.lo: one rounding of the rotated operands to bf16
// would put an error of ~2^-9 |q||k| into every score (a GDPA output sums such errors without
// normalisation), the split leaves ~2^-17. Rows n .. 63 of the lo tiles are cleared (the hi rows
// there are finite copies of row 0, masked later).
// Thread t of NTH takes row t / (NTH / 64) and the 16-byte chunks k0 .. k0 + CH - 1 of it.
template <int NTH>
__device__ __forceinline__ void rope_tiles(GDPA_LDS char* sq, GDPA_LDS char* sk, GDPA_LDS char* sql,
                                           GDPA_LDS char* skl, int n, int p0,
                                           const GDPA_LDS double* c, int tid) {
  constexpr int TPR = NTH / BL;
  constexpr int CH = (D / 8) / TPR;
  const int r = tid / TPR, k0 = (tid % TPR) * CH;
  if (r >= n) {
#pragma unroll
    for (int k = k0; k < k0 + CH; ++k) {
      *(GDPA_LDS bf16x8*)(sql + xoff(r, k)) = zero_bf16x8();
      *(GDPA_LDS bf16x8*)(skl + xoff(r, k)) = zero_bf16x8();
    }
    return;
  }
#pragma unroll
  for (int k = k0; k < k0 + CH; ++k) {
    GDPA_LDS bf16x8* pq = (GDPA_LDS bf16x8*)(sq + xoff(r, k));
    GDPA_LDS bf16x8* pk = (GDPA_LDS bf16x8*)(sk + xoff(r, k));
    const bf16x8 q = *pq, kk = *pk;
    float qf[8], kf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs;
      rope_sc(c[4 * k + e], p0 + r, sn, cs);
      const float qe = (float)q[2 * e], qo = (float)q[2 * e + 1];
      const float ke = (float)kk[2 * e], ko = (float)kk[2 * e + 1];
      qf[2 * e] = cs * qe - sn * qo;
      qf[2 * e + 1] = sn * qe + cs * qo;
      kf[2 * e] = cs * ke - sn * ko;
      kf[2 * e + 1] = sn * ke + cs * ko;
    }
    const bf16x8 qh = pack8(qf), kh = pack8(kf);
    float ql[8], kl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ql[e] = qf[e] - (float)qh[e];
      kl[e] = kf[e] - (float)kh[e];
    }
    *pq = qh;
    *pk = kh;
    *(GDPA_LDS bf16x8*)(sql + xoff(r, k)) = pack8(ql);
    *(GDPA_LDS bf16x8*)(skl + xoff(r, k)) = pack8(kl);
  }
}

// The forward's version of rope_tiles for K alone (its Q is rotated in registers, rope_q_regs).
template <int NTH>
__device__ __forceinline__ void rope_k_tile(GDPA_LDS char* sk, GDPA_LDS char* skl, int n, int p0,
                                            const GDPA_LDS double* c, int tid) {
  constexpr int TPR = NTH / BL;
  constexpr int CH = (D / 8) / TPR;
  const int r = tid / TPR, k0 = (tid % TPR) * CH;
  if (r >= n) {
#pragma unroll
    for (int k = k0; k < k0 + CH; ++k) *(GDPA_LDS bf16x8*)(skl + xoff(r, k)) = zero_bf16x8();
    return;
  }
#pragma unroll
  for (int k = k0; k < k0 + CH; ++k) {
    GDPA_LDS bf16x8* pk = (GDPA_LDS bf16x8*)(sk + xoff(r, k));
    const bf16x8 kk = *pk;
    float kf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs;
      rope_sc(c[4 * k + e], p0 + r, sn, cs);
      const float ke = (float)kk[2 * e], ko = (float)kk[2 * e + 1];
      kf[2 * e] = cs * ke - sn * ko;
      kf[2 * e + 1] = sn * ke + cs * ko;
    }
    const bf16x8 kh = pack8(kf);
    float kl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kl[e] = kf[e] - (float)kh[e];
    *pk = kh;
    *(GDPA_LDS bf16x8*)(skl + xoff(r, k)) = pack8(kl);
  }
}

// A lane's Q operands (query row at position pos; register s holds D indices 16s + 8g .. + 7,
// the pairs m = 8s + 4g + 0..3) rotated in registers as hi and lo parts, the same arithmetic as
// rope_tiles.
__device__ __forceinline__ void rope_q_regs(bf16x8* qop, bf16x8* qlo, int pos, int g,
                                            const GDPA_LDS double* c) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const bf16x8 q = qop[s];
    float qf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs;
      rope_sc(c[8 * s + 4 * g + e], pos, sn, cs);
      const float qe = (float)q[2 * e], qo = (float)q[2 * e + 1];
      qf[2 * e] = cs * qe - sn * qo;
      qf[2 * e + 1] = sn * qe + cs * qo;
    }
    const bf16x8 qh = pack8(qf);
    float ql[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ql[e] = qf[e] - (float)qh[e];
    qop[s] = qh;
    qlo[s] = pack8(ql);
  }
}

// Turn a lane's fp32 gradient row back (the transpose of the rotation): register r of block n
// holds D index 32n + 8(r/4) + 4g + r%4, so registers (r, r+1), r%4 in {0, 2}, are the pair
// m = 16n + 4(r/4) + 2g + (r%4)/2 of the row at position pos.
__device__ __forceinline__ void rope_back(f32x16* acc, int pos, int g, const GDPA_LDS double* c) {
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int m = 16 * n + 4 * (r >> 2) + 2 * g + ((r & 3) >> 1);
      float sn, cs;
      rope_sc(c[m], pos, sn, cs);
      const float ge = acc[n][r], go = acc[n][r + 1];
      acc[n][r] = cs * ge + sn * go;
      acc[n][r + 1] = cs * go - sn * ge;
    }
}

// The workgroup's item (sample b, block t, head h, the sample's first row and length); the item
// and the header come in one round trip (the item slot is in bounds whatever the count).
__device__ __forceinline__ bool item_of(const BlockArgs& a, int& b, int& t, int& h, int& base, int& L) {
  Item it;
  if (!fetch_item(a.hdr, a.items, 0, it)) return false;
  b = it.b;
  t = it.tile;
  h = it.h;
  base = it.q0;
  L = it.lq;
  return true;
}

// ------------------------------------------------------------------------------------------
// forward: 2 waves of 32 queries each. Q goes straight to registers (rotated there), so the
// workgroup holds only the K (hi, lo) and V tiles in LDS: 48 KiB, three workgroups per compute
// unit.
template <int ACT, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(128) void block_fwd_kernel(BlockArgs a) {
  __shared__ __attribute__((aligned(16))) char sk_[TILE];
  __shared__ __attribute__((aligned(16))) char sv_[TILE];
  __shared__ __attribute__((aligned(16))) char skl_[ROPE ? TILE : 16];
  __shared__ double c_[ROPE ? D / 2 : 1];
  GDPA_LDS char* sk = (GDPA_LDS char*)sk_;
  GDPA_LDS char* sv = (GDPA_LDS char*)sv_;
  GDPA_LDS char* skl = (GDPA_LDS char*)skl_;
  GDPA_LDS double* c = (GDPA_LDS double*)c_;
  int b, t, h;
  int base, L;
  if (!item_of(a, b, t, h, base, L)) return;
  const int H = a.H;
  const int r0 = t * BL, n = min(BL, L - r0);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // each wave issues the loads of two of the four row groups of a tile
  for (int u = w; u < 4; u += 2) {
    issue_tile(sk, (const __bf16*)a.K, r0, L, base, H, h, u, lane);
    issue_tile(sv, (const __bf16*)a.V, r0, L, base, H, h, u, lane);
  }
  const int iq = w * 32 + l32;  // the lane's query inside the block
  const bool qv = iq < n;
  bf16x8 qop[D / 16], qlo[D / 16];
  {
    const __bf16* Q = (const __bf16*)a.Q + ((int64_t)(base + r0 + (qv ? iq : 0)) * H + h) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = qv ? *(const bf16x8*)(Q + 16 * s + 8 * g) : zero_bf16x8();
  }
  if (ROPE) rope_table(c, a.rope_log2_base, tid);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ROPE) {
    rope_k_tile<128>(sk, skl, n, r0, c, tid);
    rope_q_regs(qop, qlo, r0 + iq, g, c);
    __syncthreads();
  }
  if (w * 32 >= n) return;
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      sacc[kb] = mfma32(row_op(sk, kb * 32, s, lane), qop[s], sacc[kb]);
      if (ROPE) {
        sacc[kb] = mfma32(row_op(skl, kb * 32, s, lane), qop[s], sacc[kb]);
        sacc[kb] = mfma32(row_op(sk, kb * 32, s, lane), qlo[s], sacc[kb]);
      }
    }
  // register r of half kb is key kb*32 + 8(r/4) + 4g + r%4: valid below lim[kb]
  int lim[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int l = n - kb * 32;
    if (CAUSAL) l = min(l, iq - kb * 32 + 1);
    lim[kb] = l - 4 * g;
  }
  auto valid = [&](int kb, int r) { return (r >> 2) * 8 + (r & 3) < lim[kb]; };
  float p[2][16];
  float inv = 1.0f;
  if (ACT == ACT_SOFTMAX) {
    const float sl2 = a.scale * LOG2E;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (valid(kb, r)) mt = fmaxf(mt, sacc[kb][r]);
    mt = half_max(mt) * sl2;
    const float m = mt == -INFINITY ? 0.0f : mt;
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kb][r] = valid(kb, r) ? fast_exp2(fmaf(sacc[kb][r], sl2, -m)) : 0.0f;
        ls += p[kb][r];
      }
    const float l = half_sum(ls);
    inv = l > 0.0f ? 1.0f / l : 0.0f;
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[kb][r] = valid(kb, r) ? act_fwd(ACT, sacc[kb][r] * a.scale) : 0.0f;
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int nn = 0; nn < D / 32; ++nn) o[nn] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 pb = pack8(&p[kb][8 * s2]);
#pragma unroll
      for (int nn = 0; nn < D / 32; ++nn) o[nn] = mfma32(tr_op(sv, kb * 32 + 16 * s2, nn, lane), pb, o[nn]);
    }
  if (iq >= n) return;
  __bf16* orow = (__bf16*)a.O + ((int64_t)(base + r0 + iq) * H + h) * D;
#pragma unroll
  for (int nn = 0; nn < D / 32; ++nn) store_acc_row_bf16(orow, o[nn], nn, g, inv);
}

// ------------------------------------------------------------------------------------------
// backward: waves 0-1 lane = query (dQ, row terms), waves 2-3 lane = key (dK, dV)
template <int ACT, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(256) void block_bwd_kernel(BlockArgs a) {
  constexpr bool SM = ACT == ACT_SOFTMAX;
  __shared__ __attribute__((aligned(16))) char sq_[TILE];
  __shared__ __attribute__((aligned(16))) char sk_[TILE];
  __shared__ __attribute__((aligned(16))) char sv_[TILE];
  __shared__ __attribute__((aligned(16))) char so_[TILE];
  __shared__ __attribute__((aligned(16))) char sql_[ROPE ? TILE : 16];
  __shared__ __attribute__((aligned(16))) char skl_[ROPE ? TILE : 16];
  __shared__ __attribute__((aligned(16))) float rt_[2 * BL];  // [log2-sum-exp, D_i][query]
  __shared__ double c_[ROPE ? D / 2 : 1];
  GDPA_LDS char* sq = (GDPA_LDS char*)sq_;
  GDPA_LDS char* sk = (GDPA_LDS char*)sk_;
  GDPA_LDS char* sv = (GDPA_LDS char*)sv_;
  GDPA_LDS char* so = (GDPA_LDS char*)so_;
  GDPA_LDS char* sql = (GDPA_LDS char*)sql_;
  GDPA_LDS char* skl = (GDPA_LDS char*)skl_;
  GDPA_LDS float* rt = (GDPA_LDS float*)rt_;
  GDPA_LDS double* c = (GDPA_LDS double*)c_;
  int b, t, h;
  int base, L;
  if (!item_of(a, b, t, h, base, L)) return;
  const int H = a.H;
  const int r0 = t * BL, n = min(BL, L - r0);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  issue_tile(sq, (const __bf16*)a.Q, r0, L, base, H, h, w, lane);
  issue_tile(sk, (const __bf16*)a.K, r0, L, base, H, h, w, lane);
  issue_tile(sv, (const __bf16*)a.V, r0, L, base, H, h, w, lane);
  issue_tile(so, (const __bf16*)a.dO, r0, L, base, H, h, w, lane);
  if (ROPE) rope_table(c, a.rope_log2_base, tid);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ROPE) {
    rope_tiles<256>(sq, sk, sql, skl, n, r0, c, tid);
    __syncthreads();
  }
  const float sc = SM ? a.scale * LOG2E : a.scale;

  if (w < 2) {
    // ---- lane = query iq; registers of half kb are keys kb*32 + 8(r/4) + 4g + r%4
    const int iq = w * 32 + l32;
    f32x16 dq[D / 32];
#pragma unroll
    for (int nn = 0; nn < D / 32; ++nn) dq[nn] = f32x16{};
    if (w * 32 < n) {
      f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
      {
        bf16x8 qop[D / 16], qlo[D / 16], dop[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          qop[s] = row_op(sq, w * 32, s, lane);
          if (ROPE) qlo[s] = row_op(sql, w * 32, s, lane);
          dop[s] = row_op(so, w * 32, s, lane);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < D / 16; ++s) {
            sacc[kb] = mfma32(row_op(sk, kb * 32, s, lane), qop[s], sacc[kb]);
            if (ROPE) {
              sacc[kb] = mfma32(row_op(skl, kb * 32, s, lane), qop[s], sacc[kb]);
              sacc[kb] = mfma32(row_op(sk, kb * 32, s, lane), qlo[s], sacc[kb]);
            }
            dpacc[kb] = mfma32(row_op(sv, kb * 32, s, lane), dop[s], dpacc[kb]);
          }
      }
      int lim[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        int l = n - kb * 32;
        if (CAUSAL) l = min(l, iq - kb * 32 + 1);
        lim[kb] = l - 4 * g;
      }
      auto valid = [&](int kb, int r) { return (r >> 2) * 8 + (r & 3) < lim[kb]; };
      float ds[2][16];
      if (SM) {
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (valid(kb, r)) mt = fmaxf(mt, sacc[kb][r]);
        mt = half_max(mt) * sc;
        const float m = mt == -INFINITY ? 0.0f : mt;
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            ds[kb][r] = valid(kb, r) ? fast_exp2(fmaf(sacc[kb][r], sc, -m)) : 0.0f;  // e^(s - m)
            ls += ds[kb][r];
          }
        const float l = half_sum(ls);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float di = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            ds[kb][r] *= inv;  // p
            di = fmaf(ds[kb][r], dpacc[kb][r], di);
          }
        di = half_sum(di);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[kb][r] = ds[kb][r] * (dpacc[kb][r] - di);
        if (g == 0) {
          rt[iq] = l > 0.0f ? m + log2f(l) : 0.0f;
          rt[BL + iq] = di;
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float y, dy;
            act_fwd_bwd(ACT, sacc[kb][r] * sc, y, dy);
            ds[kb][r] = valid(kb, r) ? dpacc[kb][r] * dy : 0.0f;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 db = pack8(&ds[kb][8 * s2]);
#pragma unroll
          for (int nn = 0; nn < D / 32; ++nn) {
            dq[nn] = mfma32(tr_op(sk, kb * 32 + 16 * s2, nn, lane), db, dq[nn]);
            if (ROPE) dq[nn] = mfma32(tr_op(skl, kb * 32 + 16 * s2, nn, lane), db, dq[nn]);
          }
        }
    }
    __syncthreads();  // row terms are in LDS for waves 2-3
    if (iq >= n) return;
    if (ROPE) rope_back(dq, r0 + iq, g, c);
    __bf16* qrow = (__bf16*)a.dQ + ((int64_t)(base + r0 + iq) * H + h) * D;
#pragma unroll
    for (int nn = 0; nn < D / 32; ++nn) store_acc_row_bf16(qrow, dq[nn], nn, g, a.scale);
    return;
  }

  // ---- lane = key jk; registers of query half qb are queries qb*32 + 8(r/4) + 4g + r%4
  // The score and dP products need no row terms: they run while waves 0-1 form them, and only
  // the gradient arithmetic waits for the barrier.
  const int kw = w - 2;
  const int jk = kw * 32 + l32;
  const bool kact = kw * 32 < n;
  auto half_on = [&](int qb) { return qb * 32 < n && !(CAUSAL && qb * 32 + 31 < kw * 32); };
  f32x16 sacc2[2], dpacc2[2];
  if (kact) {
    bf16x8 kop[D / 16], klo[D / 16], vop[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kop[s] = row_op(sk, kw * 32, s, lane);
      if (ROPE) klo[s] = row_op(skl, kw * 32, s, lane);
      vop[s] = row_op(sv, kw * 32, s, lane);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc2[qb] = f32x16{};
      dpacc2[qb] = f32x16{};
      if (!half_on(qb)) continue;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc2[qb] = mfma32(row_op(sq, qb * 32, s, lane), kop[s], sacc2[qb]);
        if (ROPE) {
          sacc2[qb] = mfma32(row_op(sql, qb * 32, s, lane), kop[s], sacc2[qb]);
          sacc2[qb] = mfma32(row_op(sq, qb * 32, s, lane), klo[s], sacc2[qb]);
        }
        dpacc2[qb] = mfma32(row_op(so, qb * 32, s, lane), vop[s], dpacc2[qb]);
      }
    }
  }
  __syncthreads();  // waves 0-1 have written the row terms
  if (!kact) return;
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int nn = 0; nn < D / 32; ++nn) {
    dk[nn] = f32x16{};
    dv[nn] = f32x16{};
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!half_on(qb)) continue;
    const f32x16 sacc = sacc2[qb], dpacc = dpacc2[qb];
    const int ib = qb * 32 + 4 * g;  // query of register r: ib + 8(r/4) + r%4
    float pv[16], dsv[16];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      f32x4 l4 = {}, d4 = {};
      if (SM) {
        l4 = *(const GDPA_LDS f32x4*)(rt + ib + m4 * 8);
        d4 = *(const GDPA_LDS f32x4*)(rt + BL + ib + m4 * 8);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * m4 + e;
        const int i = ib + m4 * 8 + e;
        const bool ok = i < n && jk < n && (!CAUSAL || jk <= i);
        float p, d;
        if (SM) {
          p = fast_exp2(fmaf(sacc[r], sc, -l4[e]));
          d = p * (dpacc[r] - d4[e]);
        } else {
          float dy;
          act_fwd_bwd(ACT, sacc[r] * sc, p, dy);
          d = dpacc[r] * dy;
        }
        pv[r] = ok ? p : 0.0f;
        dsv[r] = ok ? d : 0.0f;
      }
    }
    const bf16x8 pb0 = pack8(&pv[0]), pb1 = pack8(&pv[8]);
    const bf16x8 db0 = pack8(&dsv[0]), db1 = pack8(&dsv[8]);
#pragma unroll
    for (int nn = 0; nn < D / 32; ++nn) {
      dv[nn] = mfma32(tr_op(so, qb * 32, nn, lane), pb0, dv[nn]);
      dv[nn] = mfma32(tr_op(so, qb * 32 + 16, nn, lane), pb1, dv[nn]);
      dk[nn] = mfma32(tr_op(sq, qb * 32, nn, lane), db0, dk[nn]);
      dk[nn] = mfma32(tr_op(sq, qb * 32 + 16, nn, lane), db1, dk[nn]);
      if (ROPE) {
        dk[nn] = mfma32(tr_op(sql, qb * 32, nn, lane), db0, dk[nn]);
        dk[nn] = mfma32(tr_op(sql, qb * 32 + 16, nn, lane), db1, dk[nn]);
      }
    }
  }
  if (jk >= n) return;
  if (ROPE) rope_back(dk, r0 + jk, g, c);
  const int64_t krow = ((int64_t)(base + r0 + jk) * H + h) * D;
#pragma unroll
  for (int nn = 0; nn < D / 32; ++nn) {
    store_acc_row_bf16((__bf16*)a.dK + krow, dk[nn], nn, g, a.scale);
    store_acc_row_bf16((__bf16*)a.dV + krow, dv[nn], nn, g, 1.0f);
  }
}

template <int ACT, bool CAUSAL, bool ROPE>
hipError_t launch_t(const BlockArgs& a, int grid, bool bwd, hipStream_t s) {
  if (bwd) {
    prof_before(PROF_BLOCK_BWD, s);
    hipLaunchKernelGGL((block_bwd_kernel<ACT, CAUSAL, ROPE>), dim3(grid), dim3(256), 0, s, a);
    prof_after(PROF_BLOCK_BWD, s);
  } else {
    prof_before(PROF_BLOCK_FWD, s);
    hipLaunchKernelGGL((block_fwd_kernel<ACT, CAUSAL, ROPE>), dim3(grid), dim3(128), 0, s, a);
    prof_after(PROF_BLOCK_FWD, s);
  }
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_a(bool causal, bool rope, const BlockArgs& a, int grid, bool bwd, hipStream_t s) {
  if (causal) return rope ? launch_t<ACT, true, true>(a, grid, bwd, s) : launch_t<ACT, true, false>(a, grid, bwd, s);
  return rope ? launch_t<ACT, false, true>(a, grid, bwd, s) : launch_t<ACT, false, false>(a, grid, bwd, s);
}

}  // namespace blk

hipError_t launch_block(int act, bool causal, bool rope, const BlockArgs& a, int grid, bool bwd,
                        hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (act) {
    case ACT_SOFTMAX: return blk::launch_a<ACT_SOFTMAX>(causal, rope, a, grid, bwd, s);
    case ACT_GELU_TANH: return blk::launch_a<ACT_GELU_TANH>(causal, rope, a, grid, bwd, s);
    default: return blk::launch_a<ACT_SILU>(causal, rope, a, grid, bwd, s);
  }
}

}  // namespace gdpa
