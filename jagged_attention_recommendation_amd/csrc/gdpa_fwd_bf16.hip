// Forward kernel, bf16 inputs, fp32 accumulation: JFA (softmax) and GDPA (GELU-tanh / SiLU).
//
// Method (page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
// Model"): JFA paragraph - FlashAttention run directly on jagged tensors (no padding), with
// attention biases and different query / key lengths; GDPA paragraph - the same two products
// with an element-wise GELU or SiLU instead of softmax and no normalisation. FlashAttention's
// tiling with online max / sum rescaling gives exactly the plain softmax result; GDPA needs no
// rescaling since every score is mapped on its own.
//
// Work decomposition: one workgroup (4 waves) per scheduler item = 128 query rows of one
// (sample, head). Each wave owns 32 queries. Keys stream through LDS in tiles of 64 rows; the
// next tile's global loads are issued before the current tile is computed.
//
// Operand choice (wave64 MFMA 32x32x16 bf16):
//   S^T = K Q^T  : A = K rows from LDS (row-major, 16-byte reads), B = Q^T from registers. The
//                  accumulator puts one query per lane (column) and 16 keys per lane (rows), so
//                  row statistics need only a swap between the two half-waves.
//   O^T += V^T P^T: A = V^T read transposed from the row-major V tile (ds_read_b64_tr_b16),
//                  B = P^T straight from the S^T accumulator (the key order inside a 16-key
//                  k-step is permuted identically on both operands).
// The exp of softmax uses exp2 with log2(e) folded into the score scale.
#include <math.h>

#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

namespace {

constexpr int BM = FWD_BM_BF16;  // queries per item (4 waves x 32)
constexpr int BN = FWD_BN_BF16;  // keys per tile

template <int D>
struct FwdTile {
  // K tile: row pitch = 2D + 16 bytes so the 16 rows read by 16 lanes fall in distinct banks.
  static constexpr int KP = 2 * D + 16;
  // V tile: the transposed read touches 4 rows x 64 bytes per half-wave; a pitch = 64 mod 256
  // bytes spreads them over all banks.
  static constexpr int VP = D == 32 ? 192 : 2 * D + 64;
  static constexpr int K_BYTES = BN * KP;
  static constexpr int V_BYTES = BN * VP;
  static constexpr int CHUNKS = BN * D / 8;    // 16-byte chunks per tile
  static constexpr int PER_THREAD = CHUNKS / 256;
};

template <int D, int ACT, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  static_assert(T::PER_THREAD >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) char smem[T::K_BYTES + T::V_BYTES];
  GDPA_LDS char* Ks = (GDPA_LDS char*)smem;
  GDPA_LDS char* Vs = Ks + T::K_BYTES;

  const WsHeader* hdr = (const WsHeader*)a.hdr;
  if (hdr->error != 0 || (int)blockIdx.x >= hdr->n_items) return;
  const Item it = ((const Item*)a.items)[blockIdx.x];
  const int b = it.b, h = it.h, H = a.H;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lk = a.kv_off[b + 1] - kv0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int row_blk = it.tile * BM;               // first query of the item (local index)
  const int wrow = row_blk + w * 32;              // first query of this wave
  const int iq = wrow + l32;                      // this lane's query
  const bool wave_active = wrow < Lq;

  const __bf16* Q = (const __bf16*)a.Q;
  const __bf16* K = (const __bf16*)a.K;
  const __bf16* V = (const __bf16*)a.V;

  // number of key tiles this item visits
  int nkt = (Lk + BN - 1) / BN;
  if (CAUSAL) {
    int i_max = min(Lq, row_blk + BM) - 1;
    nkt = min(nkt, i_max / BN + 1);
  }

  // Q^T operand: lane holds query iq, d = 16*s + 8*g .. +8
  bf16x8 qop[D / 16];
  {
    const bool qv = iq < Lq;
    const __bf16* qrow = Q + ((int64_t)(q0 + (qv ? iq : 0)) * H + h) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qop[s] = qv ? *(const bf16x8*)(qrow + 16 * s + 8 * g) : zero_bf16x8();
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = a.scale * LOG2E;
  const float* bias_h = BIAS ? a.bias + (int64_t)h * a.nb : nullptr;

  // global -> register prefetch of one K/V tile
  i32x4 pk[T::PER_THREAD], pv[T::PER_THREAD];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; ++u) {
      int c = tid + 256 * u;
      int r = c / (D / 8), col = c % (D / 8);
      int j = kt * BN + r;
      if (j < Lk) {
        int64_t off = ((int64_t)(kv0 + j) * H + h) * D + col * 8;
        pk[u] = *(const i32x4*)(K + off);
        pv[u] = *(const i32x4*)(V + off);
      } else {
        pk[u] = i32x4{0, 0, 0, 0};
        pv[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; ++u) {
      int c = tid + 256 * u;
      int r = c / (D / 8), col = c % (D / 8);
      *(GDPA_LDS i32x4*)(Ks + r * T::KP + col * 16) = pk[u];
      *(GDPA_LDS i32x4*)(Vs + r * T::VP + col * 16) = pv[u];
    }
  };

  if (nkt > 0) prefetch(0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kt + 1 < nkt) prefetch(kt + 1);
    const int k0 = kt * BN;
    if (!wave_active) continue;
    if (CAUSAL && k0 > wrow + 31) continue;  // every key of the tile is after every query

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const GDPA_LDS char* krow = Ks + (kb * 32 + l32) * T::KP + 16 * g;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        bf16x8 ka = *(const GDPA_LDS bf16x8*)(krow + 32 * s);
        sacc[kb] = mfma32(ka, qop[s], sacc[kb]);
      }
    }

    // ---- scores -> probabilities (register r of block kb is key k0 + kb*32 + (r/4)*8 + 4g + r%4)
    const bool need_mask = (k0 + BN > Lk) || (CAUSAL && k0 + BN - 1 > wrow);
    float p[2][16];
    if (ACT == ACT_SOFTMAX) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
          float x = sacc[kb][r] * sl2;
          if (BIAS) x += bias_h[clampi(iq - j, 0, a.nb - 1)] * LOG2E;
          if (need_mask && (j >= Lk || (CAUSAL && j > iq))) x = -INFINITY;
          p[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = half_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[kb][r] = fast_exp2(p[kb][r] - m_use);
          ls += p[kb][r];
        }
      }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int n = 0; n < D / 32; ++n) o[n] *= alpha;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3);
          float x = sacc[kb][r] * a.scale;
          if (BIAS) x += bias_h[clampi(iq - j, 0, a.nb - 1)];
          float y = act_fwd(ACT, x);
          if (need_mask && (j >= Lk || (CAUSAL && j > iq))) y = 0.0f;
          p[kb][r] = y;
        }
      }
    }

    // ---- O^T += V^T P^T
    const int i16 = lane & 15, tq = i16 >> 2, qq = i16 & 3;
    const int dsub = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(&p[kb][8 * s2]);
        const int key0 = kb * 32 + 16 * s2 + 4 * g;
        const GDPA_LDS char* v_lo = Vs + (key0 + tq) * T::VP + (dsub + 4 * qq) * 2;
        const GDPA_LDS char* v_hi = v_lo + 8 * T::VP;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
          const bf16x8 va = cat_tr(lds_read_tr(v_lo + n * 64), lds_read_tr(v_hi + n * 64));
          o[n] = mfma32(va, pb, o[n]);
        }
      }
    }
  }

  if (!wave_active) return;
  // ---- epilogue: lane owns query iq; register r of block n is d = n*32 + (r/4)*8 + 4g + r%4
  const bool qv = iq < Lq;
  float inv = 1.0f;
  if (ACT == ACT_SOFTMAX) {
    const float lt = half_sum(l_run);
    inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qv && g == 0 && a.lse != nullptr) {
      a.lse[(int64_t)(q0 + iq) * H + h] = lt > 0.0f ? (m_run + log2f(lt)) * LN2 : -INFINITY;
    }
  }
  if (!qv) return;
  __bf16* orow = (__bf16*)a.O + ((int64_t)(q0 + iq) * H + h) * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x2 lo = pack_bf16(o[n][4 * r4 + 0] * inv, o[n][4 * r4 + 1] * inv);
      bf16x2 hi = pack_bf16(o[n][4 * r4 + 2] * inv, o[n][4 * r4 + 3] * inv);
      bf16x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
      *(bf16x4*)(orow + n * 32 + r4 * 8 + 4 * g) = v4;
    }
  }
}

template <int D, int ACT, bool CAUSAL, bool BIAS>
hipError_t launch_t(const FwdArgs& a, int grid, hipStream_t s) {
  prof_before(PROF_FWD, s);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ACT, CAUSAL, BIAS>), dim3(grid), dim3(256), 0, s, a);
  prof_after(PROF_FWD, s);
  return hipGetLastError();
}

template <int D, int ACT>
hipError_t launch_cb(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  const bool bias = p.nb > 0;
  if (p.causal) return bias ? launch_t<D, ACT, true, true>(a, grid, s) : launch_t<D, ACT, true, false>(a, grid, s);
  return bias ? launch_t<D, ACT, false, true>(a, grid, s) : launch_t<D, ACT, false, false>(a, grid, s);
}

template <int D>
hipError_t launch_d(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  switch (p.act) {
    case ACT_SOFTMAX: return launch_cb<D, ACT_SOFTMAX>(p, a, grid, s);
    case ACT_GELU_TANH: return launch_cb<D, ACT_GELU_TANH>(p, a, grid, s);
    default: return launch_cb<D, ACT_SILU>(p, a, grid, s);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (p.D) {
    case 32: return launch_d<32>(p, a, grid, s);
    case 64: return launch_d<64>(p, a, grid, s);
    default: return launch_d<128>(p, a, grid, s);
  }
}

}  // namespace gdpa
