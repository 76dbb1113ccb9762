/*
 * Reference oracle for jagged attention (JFA softmax and GDPA activation attention).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, fp64 definition that the GPU
 * library is checked against. Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the product path never does. It shares no code, header, table or
 * helper with the HIP library.
 *
 * What is computed (sources: the page "GEM Training: How Meta Doubled the Efficiency of Its
 * LLM-Scale Ads Foundation Model", custom-kernel-library part):
 *   - JFA paragraph: FlashAttention applied directly to variable-length (jagged) tensors, with
 *     custom attention biases, different query and key/value lengths, and backward passes.
 *     FlashAttention reaches exactly the plain softmax attention result, so this oracle is that
 *     plain definition (no tiling, no online rescaling).
 *   - GDPA paragraph: the same two matrix products with an element-wise activation (GELU or
 *     SiLU) in place of softmax, with no normalisation.
 *   - Block-attention paragraph: it names the logsumexp and the "Di" row term of the softmax
 *     backward; lse_i = m_i + ln l_i and D_i = sum_j p_ij dp_ij are those quantities.
 *
 * Definition, per sample b and head h, local query i in [0,Lq) and key j in [0,Lk):
 *   valid(i,j) = (!causal || j <= i) && (W == 0 || j > i - W)
 *     W >= 1 is a sliding window (same page, self-attention paragraph on sliding-window
 *     attention: each token attends only to nearby events; read as the W most recent keys,
 *     itself included); the library takes it with causal = 1
 *   s_ij = scale * <q_i,k_j> + bias[h, clamp(i-j, 0, NB-1)]        (bias term absent if NB = 0)
 *   softmax: p_ij = exp(s_ij - m_i) / l_i over valid j, o_i = sum_j p_ij v_j, lse_i = m_i + ln l_i
 *            a row with no valid key gives o_i = 0, lse_i = -inf
 *   GDPA:    p_ij = act(s_ij) for valid j, else 0; o_i = sum_j p_ij v_j (no normalisation)
 *   backward, given dO:
 *     dp_ij = <do_i, v_j>
 *     softmax: ds_ij = p_ij (dp_ij - D_i), D_i = sum_j p_ij dp_ij
 *     GDPA:    ds_ij = dp_ij act'(s_ij)
 *     dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij do_i
 *     dbias[h,r] = sum over b and valid (i,j) with clamp(i-j,0,NB-1) = r of ds_ij
 *   error scale of dbias (optional output, not a result): a low-precision softmax backward forms
 *   D_i from a forward output that carries rounding. Each rounding multiplies the value it rounds
 *   by (1 + delta), with independent zero-mean deltas of standard deviation eps: one per
 *   probability p_ij, rounded once before the product with V (so the same delta reaches every
 *   column c of o_i), and one per element o_ic when the output is stored. Then
 *     delta D_i = sum_j delta_ij p_ij dp_ij + sum_c delta'_ic do_ic o_ic,
 *   of variance eps^2 w_i with
 *     w_i = sum_j p_ij^2 dp_ij^2 + sum_c do_ic^2 o_ic^2,
 *   and since ds_ij = p_ij (dp_ij - D_i), bucket r moves by -sum_i m_ir delta D_i, where m_ir is
 *   the sum of p_ij over the row's pairs in r: variance eps^2 sum_i m_ir^2 w_i.
 *   dbias_scale[h,r] = sqrt(sum over b, i of m_ir^2 w_i) (0 for GDPA, which has no D_i).
 *   Buckets that sum whole rows cancel (softmax rows of ds sum to 0), so this term, not |dbias|,
 *   sets how close a rounded backward can come there.
 *   gelu_tanh(x) = x/2 (1 + tanh(c (x + a x^3))), c = sqrt(2/pi), a = 0.044715
 *   silu(x)      = x sigmoid(x)
 *
 * MX decode (OCP Microscaling Formats v1.0): an e4m3 element is sign, 4 exponent bits with
 * bias 7 and 3 mantissa bits, exponent 0 is subnormal, S.1111.111 is NaN and there is no
 * infinity; an e8m0 scale X means 2^(X-127), with 0xFF = NaN. A block of 32 consecutive
 * elements along the head dimension shares one scale.
 *
 * Layout: Q/O/dQ are [total_q, H, D] row-major doubles, K/V/dK/dV are [total_kv, H, D],
 * lse and Dvec are [total_q, H], bias and dbias are [H, NB]. Offsets are int32 prefix sums of
 * length B+1. Parallel over (sample, head) with OpenMP; every output element is produced by a
 * single (sample, head) task, and dbias is reduced over samples in sample order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ACT_SOFTMAX 0
#define ORACLE_ACT_GELU_TANH 1
#define ORACLE_ACT_SILU 2

static const double GELU_C = 0.79788456080286535588; /* sqrt(2/pi) */
static const double GELU_A = 0.044715;

static double act_value(int act, double x) {
  if (act == ORACLE_ACT_GELU_TANH) {
    double u = GELU_C * (x + GELU_A * x * x * x);
    return 0.5 * x * (1.0 + tanh(u));
  }
  /* silu */
  return x / (1.0 + exp(-x));
}

static double act_deriv(int act, double x) {
  if (act == ORACLE_ACT_GELU_TANH) {
    double u = GELU_C * (x + GELU_A * x * x * x);
    double t = tanh(u);
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * x * x);
  }
  double sg = 1.0 / (1.0 + exp(-x));
  return sg * (1.0 + x * (1.0 - sg));
}

/* Exposed so the tests can pin the activations on their own. */
void gdpa_oracle_act(int act, const double* x, long n, double* y, double* dy) {
  for (long t = 0; t < n; ++t) {
    if (y) y[t] = act_value(act, x[t]);
    if (dy) dy[t] = act_deriv(act, x[t]);
  }
}

static int bias_index(long i, long j, int nb) {
  long r = i - j;
  if (r < 0) r = 0;
  if (r > nb - 1) r = nb - 1;
  return (int)r;
}

static double dot(const double* a, const double* b, int n) {
  double acc = 0.0;
  for (int c = 0; c < n; ++c) acc += a[c] * b[c];
  return acc;
}

/* Checks the offsets; returns 0 when they are non-decreasing and start at 0. */
static int check_offsets(int B, const int32_t* off) {
  if (off[0] != 0) return 1;
  for (int b = 0; b < B; ++b)
    if (off[b + 1] < off[b]) return 1;
  return 0;
}

/* Scores of one query row against every key of its sample. valid[j] marks the unmasked keys.
 * Returns the number of valid keys. */
static long row_scores(int D, int H, int h, long i, long Lk, const double* qi, const double* Kb,
                       const double* bias_h, int nb, int causal, int window, double scale,
                       double* s, unsigned char* valid) {
  long nvalid = 0;
  for (long j = 0; j < Lk; ++j) {
    valid[j] = (unsigned char)((!causal || j <= i) && (window <= 0 || j > i - window));
    if (!valid[j]) continue;
    double v = scale * dot(qi, Kb + (size_t)j * H * D + (size_t)h * D, D);
    if (nb > 0) v += bias_h[bias_index(i, j, nb)];
    s[j] = v;
    ++nvalid;
  }
  return nvalid;
}

/* Probabilities p_ij of one row: softmax over the valid keys, or act(s_ij). Returns lse_i for
 * softmax (-inf when the row has no valid key), 0 otherwise. */
static double row_probs(int act, long Lk, const double* s, const unsigned char* valid, long nvalid,
                        double* p) {
  if (act != ORACLE_ACT_SOFTMAX) {
    for (long j = 0; j < Lk; ++j) p[j] = valid[j] ? act_value(act, s[j]) : 0.0;
    return 0.0;
  }
  if (nvalid == 0) {
    for (long j = 0; j < Lk; ++j) p[j] = 0.0;
    return -INFINITY;
  }
  double m = -INFINITY;
  for (long j = 0; j < Lk; ++j)
    if (valid[j] && s[j] > m) m = s[j];
  double l = 0.0;
  for (long j = 0; j < Lk; ++j) {
    p[j] = valid[j] ? exp(s[j] - m) : 0.0;
    l += p[j];
  }
  for (long j = 0; j < Lk; ++j) p[j] /= l;
  return m + log(l);
}

int gdpa_oracle_fwd(int B, int H, int D, const int32_t* q_off, const int32_t* kv_off,
                    const double* Q, const double* K, const double* V, const double* bias, int nb,
                    int act, int causal, int window, double scale, double* O, double* lse,
                    int nthreads) {
  if (B < 0 || H <= 0 || D <= 0 || nb < 0 || window < 0) return 1;
  if (act < 0 || act > 2) return 1;
  if (check_offsets(B, q_off) || check_offsets(B, kv_off)) return 1;
  long ntask = (long)B * H;
  long maxk = 0;
  for (int b = 0; b < B; ++b) {
    long lk = kv_off[b + 1] - kv_off[b];
    if (lk > maxk) maxk = lk;
  }
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    unsigned char* valid = (unsigned char*)malloc((size_t)(maxk + 1));
    if (!s || !p || !valid) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long t = 0; t < ntask; ++t) {
        int b = (int)(t / H), h = (int)(t % H);
        long q0 = q_off[b], Lq = q_off[b + 1] - q_off[b];
        long k0 = kv_off[b], Lk = kv_off[b + 1] - kv_off[b];
        const double* Kb = K + (size_t)k0 * H * D;
        const double* Vb = V + (size_t)k0 * H * D;
        const double* bias_h = nb > 0 ? bias + (size_t)h * nb : NULL;
        for (long i = 0; i < Lq; ++i) {
          size_t row = ((size_t)(q0 + i) * H + h);
          const double* qi = Q + row * D;
          long nvalid = row_scores(D, H, h, i, Lk, qi, Kb, bias_h, nb, causal, window, scale, s, valid);
          double li = row_probs(act, Lk, s, valid, nvalid, p);
          double* oi = O + row * D;
          for (int c = 0; c < D; ++c) oi[c] = 0.0;
          for (long j = 0; j < Lk; ++j) {
            if (!valid[j]) continue;
            const double* vj = Vb + (size_t)j * H * D + (size_t)h * D;
            for (int c = 0; c < D; ++c) oi[c] += p[j] * vj[c];
          }
          if (lse) lse[row] = act == ORACLE_ACT_SOFTMAX ? li : 0.0;
        }
      }
    }
    free(s);
    free(p);
    free(valid);
  }
  return bad ? 2 : 0;
}

int gdpa_oracle_bwd(int B, int H, int D, const int32_t* q_off, const int32_t* kv_off,
                    const double* Q, const double* K, const double* V, const double* dO,
                    const double* bias, int nb, int act, int causal, int window, double scale,
                    double* dQ, double* dK, double* dV, double* dbias, double* Dvec,
                    double* dbias_scale, int nthreads) {
  if (B < 0 || H <= 0 || D <= 0 || nb < 0 || window < 0) return 1;
  if (act < 0 || act > 2) return 1;
  if (check_offsets(B, q_off) || check_offsets(B, kv_off)) return 1;
  long ntask = (long)B * H;
  long maxk = 0;
  for (int b = 0; b < B; ++b) {
    long lk = kv_off[b + 1] - kv_off[b];
    if (lk > maxk) maxk = lk;
  }
  long total_kv = kv_off[B];
  memset(dK, 0, sizeof(double) * (size_t)total_kv * H * D);
  memset(dV, 0, sizeof(double) * (size_t)total_kv * H * D);
  /* one dbias partial per (sample, head) task, reduced over samples in order afterwards */
  double* dbias_part = NULL;
  double* scale_part = NULL;
  if (nb > 0 && dbias) {
    dbias_part = (double*)calloc((size_t)(ntask > 0 ? ntask : 1) * nb, sizeof(double));
    if (!dbias_part) return 2;
  }
  if (nb > 0 && dbias_scale && act == ORACLE_ACT_SOFTMAX) {
    scale_part = (double*)calloc((size_t)(ntask > 0 ? ntask : 1) * nb, sizeof(double));
    if (!scale_part) {
      free(dbias_part);
      return 2;
    }
  }
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    double* ds = (double*)malloc(sizeof(double) * (size_t)(maxk + 1));
    unsigned char* valid = (unsigned char*)malloc((size_t)(maxk + 1));
    double* pv = (double*)malloc(sizeof(double) * (size_t)D * 2);
    double* mr = (double*)calloc((size_t)(nb > 0 ? nb : 1), sizeof(double));
    if (!s || !p || !dp || !ds || !valid || !pv || !mr) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long t = 0; t < ntask; ++t) {
        int b = (int)(t / H), h = (int)(t % H);
        long q0 = q_off[b], Lq = q_off[b + 1] - q_off[b];
        long k0 = kv_off[b], Lk = kv_off[b + 1] - kv_off[b];
        const double* Kb = K + (size_t)k0 * H * D;
        const double* Vb = V + (size_t)k0 * H * D;
        const double* bias_h = nb > 0 ? bias + (size_t)h * nb : NULL;
        double* part = dbias_part ? dbias_part + (size_t)t * nb : NULL;
        double* spart = scale_part ? scale_part + (size_t)t * nb : NULL;
        for (long i = 0; i < Lq; ++i) {
          size_t row = ((size_t)(q0 + i) * H + h);
          const double* qi = Q + row * D;
          const double* doi = dO + row * D;
          long nvalid = row_scores(D, H, h, i, Lk, qi, Kb, bias_h, nb, causal, window, scale, s, valid);
          row_probs(act, Lk, s, valid, nvalid, p);
          double Di = 0.0;
          for (long j = 0; j < Lk; ++j) {
            dp[j] = 0.0;
            if (!valid[j]) continue;
            dp[j] = dot(doi, Vb + (size_t)j * H * D + (size_t)h * D, D);
            Di += p[j] * dp[j];
          }
          for (long j = 0; j < Lk; ++j) {
            if (!valid[j]) {
              ds[j] = 0.0;
              continue;
            }
            ds[j] = act == ORACLE_ACT_SOFTMAX ? p[j] * (dp[j] - Di) : dp[j] * act_deriv(act, s[j]);
          }
          if (Dvec) Dvec[row] = act == ORACLE_ACT_SOFTMAX ? Di : 0.0;
          double* dqi = dQ + row * D;
          for (int c = 0; c < D; ++c) dqi[c] = 0.0;
          for (long j = 0; j < Lk; ++j) {
            if (!valid[j]) continue;
            size_t krow = (size_t)j * H * D + (size_t)h * D;
            const double* kj = Kb + krow;
            double* dkj = dK + (size_t)k0 * H * D + krow;
            double* dvj = dV + (size_t)k0 * H * D + krow;
            for (int c = 0; c < D; ++c) {
              dqi[c] += scale * ds[j] * kj[c];
              dkj[c] += scale * ds[j] * qi[c];
              dvj[c] += p[j] * doi[c];
            }
            if (part) part[bias_index(i, j, nb)] += ds[j];
          }
          if (spart) {
            /* w_i = sum_j p_ij^2 dp_ij^2 + sum_c do_ic^2 o_ic^2; m_ir per bucket of the row */
            double* oc = pv;
            for (int c = 0; c < D; ++c) oc[c] = 0.0;
            double wi = 0.0;
            for (long j = 0; j < Lk; ++j) {
              if (!valid[j]) continue;
              const double* vj = Vb + (size_t)j * H * D + (size_t)h * D;
              for (int c = 0; c < D; ++c) oc[c] += p[j] * vj[c];
              wi += p[j] * p[j] * dp[j] * dp[j];
            }
            for (int c = 0; c < D; ++c) wi += doi[c] * doi[c] * oc[c] * oc[c];
            for (long j = 0; j < Lk; ++j)
              if (valid[j]) mr[bias_index(i, j, nb)] += p[j];
            /* the row's buckets are bias_index(i, Lk - 1) .. bias_index(i, 0) */
            for (int r = bias_index(i, Lk - 1, nb); r <= bias_index(i, 0, nb); ++r) {
              spart[r] += mr[r] * mr[r] * wi;
              mr[r] = 0.0;
            }
          }
        }
      }
    }
    free(pv);
    free(mr);
    free(s);
    free(p);
    free(dp);
    free(ds);
    free(valid);
  }
  if (dbias_part) {
    for (int h = 0; h < H; ++h)
      for (int r = 0; r < nb; ++r) {
        double acc = 0.0;
        for (int b = 0; b < B; ++b) acc += dbias_part[((size_t)b * H + h) * nb + r];
        dbias[(size_t)h * nb + r] = acc;
      }
    free(dbias_part);
  } else if (dbias && nb > 0) {
    memset(dbias, 0, sizeof(double) * (size_t)H * nb);
  }
  if (dbias_scale && nb > 0) {
    for (int h = 0; h < H; ++h)
      for (int r = 0; r < nb; ++r) {
        double acc = 0.0;
        if (scale_part)
          for (int b = 0; b < B; ++b) acc += scale_part[((size_t)b * H + h) * nb + r];
        dbias_scale[(size_t)h * nb + r] = sqrt(acc);
      }
  }
  free(scale_part);
  return bad ? 2 : 0;
}

/* e4m3 code -> value, following the OCP MX v1.0 element encoding. */
static double decode_e4m3(unsigned char code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

static double decode_e8m0(unsigned char x) {
  if (x == 0xFF) return NAN;
  return ldexp(1.0, (int)x - 127);
}

void gdpa_oracle_decode_e4m3(const unsigned char* codes, long n, double* out) {
  for (long t = 0; t < n; ++t) out[t] = decode_e4m3(codes[t]);
}

void gdpa_oracle_decode_e8m0(const unsigned char* codes, long n, double* out) {
  for (long t = 0; t < n; ++t) out[t] = decode_e8m0(codes[t]);
}

/* data: [rows, D] e4m3 codes, scales: [rows, D/32] e8m0 codes -> out [rows, D]. */
int gdpa_oracle_decode_mx(const unsigned char* data, const unsigned char* scales, long rows, int D,
                          double* out) {
  if (D <= 0 || D % 32 != 0) return 1;
  int nblk = D / 32;
  for (long r = 0; r < rows; ++r)
    for (int c = 0; c < D; ++c)
      out[(size_t)r * D + c] =
          decode_e4m3(data[(size_t)r * D + c]) * decode_e8m0(scales[(size_t)r * nblk + c / 32]);
  return 0;
}
