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

#include "gdpa_common.h"
#include "gdpa_internal.h"
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
template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(NT, 1) void dq_kernel(BwdArgs a) {
  using T = Tile<D>;
  constexpr int DSP = KL + 1;  // dS staging pitch (floats)
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BYTES + (BIAS ? QI * DSP * 4 : 0)];
  GDPA_LDS char* Ks = (GDPA_LDS char*)smem;
  GDPA_LDS char* Vs = Ks + T::BYTES;
  GDPA_LDS float* dSs = (GDPA_LDS float*)(Vs + T::BYTES);

  const WsHeader* hdr = (const WsHeader*)a.hdr;
  if (hdr->error != 0 || (int)blockIdx.x >= hdr->n_items) return;
  const Item it = ((const Item*)a.items_q)[blockIdx.x];
  const int b = it.b, h = it.h, H = a.H, nb = a.nb;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lk = a.kv_off[b + 1] - kv0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int i0 = it.tile * QI;
  const int wrow = i0 + w * 32;
  const int iq = wrow + l32;
  const bool qv = iq < Lq;
  const bool wave_active = wrow < Lq;
  const int64_t row = (int64_t)(q0 + (qv ? iq : 0)) * H + h;

  const __bf16* Q = (const __bf16*)a.Q;
  const __bf16* dO = (const __bf16*)a.dO;

  bf16x8 qop[D / 16], doop[D / 16];
  float part_d = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qop[s] = qv ? *(const bf16x8*)(Q + row * D + 16 * s + 8 * g) : zero_bf16x8();
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
      if (g == 0) a.Dvec[row] = Di;
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) dq[n] = f32x16{};

  int nkt = (Lk + KL - 1) / KL;
  if (CAUSAL) nkt = min(nkt, (min(Lq, i0 + QI) - 1) / KL + 1);
  if (i0 >= Lq) nkt = 0;

  float* part = nullptr;
  if (BIAS) {
    part = a.dbias_part + ((int64_t)it.aux * H + h) * nb;
    if (Lk > 0 && i0 < Lq) {
      const int c_lo = clampi(i0 - (Lk - 1), 0, nb - 1);
      const int c_hi = clampi(min(Lq, i0 + QI) - 1, 0, nb - 1);
      for (int c = c_lo + ((tid - c_lo % NT) % NT + NT) % NT; c <= c_hi; c += NT) part[c] = 0.0f;
    }
  }
  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;

  TileLoader<D, NT> lk_, lv_;
  if (nkt > 0) {
    lk_.load((const __bf16*)a.K, 0, Lk, kv0, H, h, tid);
    lv_.load((const __bf16*)a.V, 0, Lk, kv0, H, h, tid);
  }
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    lk_.store(Ks, tid);
    lv_.store(Vs, tid);
    __syncthreads();
    if (kt + 1 < nkt) {
      lk_.load((const __bf16*)a.K, (kt + 1) * KL, Lk, kv0, H, h, tid);
      lv_.load((const __bf16*)a.V, (kt + 1) * KL, Lk, kv0, H, h, tid);
    }
    const int k0 = kt * KL;
    const bool skip = !wave_active || (CAUSAL && k0 > wrow + 31);
    f32x16 ds_acc[2];
    if (!skip) {
      f32x16 dp_acc[2];
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
      const bool need_mask = (k0 + KL > Lk) || (CAUSAL && k0 + KL - 1 > wrow);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
          float bij = 0.0f;
          if (BIAS) bij = bias_h[clampi(iq - j, 0, nb - 1)];
          const float sraw = ds_acc[kb][r];
          float p;
          float ds = dscore<ACT>(sraw * sl2 + bij * LOG2E, sraw * a.scale + bij, lse2, Di,
                                 dp_acc[kb][r], p);
          if (!qv || (need_mask && (j >= Lk || (CAUSAL && j > iq)))) ds = 0.0f;
          ds_acc[kb][r] = ds;
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = ds_acc[kb][8 * s2 + e];
          const bf16x8 dsb = pack8(tmp);
#pragma unroll
          for (int n = 0; n < D / 32; ++n)
            dq[n] = mfma32(tile_tr_op<D>(Ks, kb * 32 + 16 * s2, n, lane), dsb, dq[n]);
        }
      }
    }
    if (BIAS) {
      // stage dS (fp32) of the whole 128 x 64 tile; rows of idle waves are zero
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dSs[(w * 32 + l32) * DSP + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3)] =
              skip ? 0.0f : ds_acc[kb][r];
      __syncthreads();
      // owner thread of clamped diagonal c is c % NT; it sums every raw diagonal rr = i - j of
      // the tile that clamps to c, in a fixed order
      int rr_lo = i0 - (k0 + KL - 1);
      const int rr_hi = i0 + QI - 1 - k0;
      if (CAUSAL) rr_lo = max(rr_lo, 0);
      if (rr_lo <= rr_hi) {
        const int c_lo = clampi(rr_lo, 0, nb - 1), c_hi = clampi(rr_hi, 0, nb - 1);
        for (int c = c_lo + ((tid - c_lo % NT) % NT + NT) % NT; c <= c_hi; c += NT) {
          const int a_lo = c == 0 ? rr_lo : c;
          const int a_hi = c == nb - 1 ? rr_hi : c;
          float acc = 0.0f;
          for (int rr = max(a_lo, rr_lo); rr <= min(a_hi, rr_hi); ++rr) {
            const int d0 = rr - (i0 - k0);  // ii - jj
            const int ii_lo = max(0, d0), ii_hi = min(QI - 1, KL - 1 + d0);
            for (int ii = ii_lo; ii <= ii_hi; ++ii) acc += dSs[ii * DSP + (ii - d0)];
          }
          part[c] += acc;
        }
      }
    }
  }
  if (!qv) return;
  __bf16* dqrow = (__bf16*)a.dQ + row * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) store_acc_row_bf16(dqrow, dq[n], n, g, a.scale);
}

// ------------------------------------------------------------------------------------------
// dK, dV
template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(NT, 1) void dkdv_kernel(BwdArgs a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BYTES + 2 * QL * 4];
  GDPA_LDS char* Qs = (GDPA_LDS char*)smem;
  GDPA_LDS char* dOs = Qs + T::BYTES;
  GDPA_LDS float* lse_s = (GDPA_LDS float*)(dOs + T::BYTES);
  GDPA_LDS float* D_s = lse_s + QL;

  const WsHeader* hdr = (const WsHeader*)a.hdr;
  if (hdr->error != 0 || (int)blockIdx.x >= hdr->n_items2) return;
  const Item it = ((const Item*)a.items_k)[blockIdx.x];
  const int b = it.b, h = it.h, H = a.H, nb = a.nb;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lk = a.kv_off[b + 1] - kv0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int j0 = it.tile * KI;
  const int wkey = j0 + w * 32;
  const int jk = wkey + l32;
  const bool kvalid = jk < Lk;
  const bool wave_active = wkey < Lk;
  const int64_t krow = (int64_t)(kv0 + (kvalid ? jk : 0)) * H + h;

  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kop[s] = kvalid ? *(const bf16x8*)((const __bf16*)a.K + krow * D + 16 * s + 8 * g) : zero_bf16x8();
    vop[s] = kvalid ? *(const bf16x8*)((const __bf16*)a.V + krow * D + 16 * s + 8 * g) : zero_bf16x8();
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }
  const int nqt = (Lq + QL - 1) / QL;
  const int qt0 = CAUSAL ? j0 / QL : 0;
  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * nb : nullptr;

  TileLoader<D, NT> lq_, ldo_;
  float st_lse = 0.0f, st_d = 0.0f;
  auto load_q = [&](int qt) {
    lq_.load((const __bf16*)a.Q, qt * QL, Lq, q0, H, h, tid);
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
    const bool need_mask = (i0 + QL > Lq) || (wkey + 32 > Lk) || (CAUSAL && i0 < wkey + 31);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(tile_row_op<D>(Qs, qb * 32, s, lane), kop[s], sacc);
        dpacc = mfma32(tile_row_op<D>(dOs, qb * 32, s, lane), vop[s], dpacc);
      }
      // register r holds query i0 + qb*32 + (r/4)*8 + 4g + r%4 for this lane's key jk
      float pv[16], dsv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ql = qb * 32 + r4 * 8 + 4 * g;
        const f32x4 l4 = *(const GDPA_LDS f32x4*)(lse_s + ql);
        const f32x4 d4 = *(const GDPA_LDS f32x4*)(D_s + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const int i = i0 + ql + e;
          float bij = 0.0f;
          if (BIAS) bij = bias_h[clampi(i - jk, 0, nb - 1)];
          float p;
          float ds = dscore<ACT>(sacc[r] * sl2 + bij * LOG2E, sacc[r] * a.scale + bij, l4[e], d4[e],
                                 dpacc[r], p);
          if (need_mask && (i >= Lq || !kvalid || (CAUSAL && jk > i))) {
            p = 0.0f;
            ds = 0.0f;
          }
          pv[r] = p;
          dsv[r] = ds;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(&pv[8 * s2]);
        const bf16x8 dsb = pack8(&dsv[8 * s2]);
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

template <int D, int ACT, bool C, bool BI>
hipError_t launch_t(const BwdArgs& a, int gq, int gk, hipStream_t s) {
  if (gq > 0) {
    prof_before(PROF_DQ, s);
    hipLaunchKernelGGL((dq_kernel<D, ACT, C, BI>), dim3(gq), dim3(NT), 0, s, a);
    prof_after(PROF_DQ, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gk > 0) {
    prof_before(PROF_DKDV, s);
    hipLaunchKernelGGL((dkdv_kernel<D, ACT, C, BI>), dim3(gk), dim3(NT), 0, s, a);
    prof_after(PROF_DKDV, s);
  }
  return hipGetLastError();
}

template <int D, int ACT>
hipError_t launch_cb(const Prob& p, const BwdArgs& a, int gq, int gk, hipStream_t s) {
  const bool bias = p.nb > 0;
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

}  // namespace

hipError_t launch_bwd_bf16(const Prob& p, const BwdArgs& a, int grid_q, int grid_k, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_d<32>(p, a, grid_q, grid_k, s);
    case 64: return launch_d<64>(p, a, grid_q, grid_k, s);
    default: return launch_d<128>(p, a, grid_q, grid_k, s);
  }
}

}  // namespace gdpa
