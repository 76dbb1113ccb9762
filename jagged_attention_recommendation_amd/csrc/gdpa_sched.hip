// Jagged work scheduler and the bias-gradient reduction.
//
// Short sequences must not leave compute units idle while long ones finish (page "GEM Training:
// How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", JFA paragraph; the GDPA
// paragraph adds that short or asymmetric K/V and large batches break occupancy assumptions and
// that scheduling was redesigned). The scheduler turns the offsets into a list of equal-shaped
// work items, one per (sample, head, tile), sorted by decreasing cost: the cost of an item is the
// number of inner-loop tiles it visits (all tiles, or only those allowed by causal masking).
// Workgroups are handed out by the hardware in index order, so the longest items start first
// and short ones fill the gaps at the end (longest-processing-time-first list scheduling).
//
// One workgroup of 1024 threads per list (the backward builds its query-tile and key-tile lists
// in one launch). Samples are walked in chunks of 1024: a scan of their tile counts gives each
// tile a canonical index, threads then take tiles (not samples) so long samples do not serialise.
// The relative order of equal-cost items is not fixed, which cannot change results: every item
// computes its outputs on its own.
#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

constexpr int NBUCKET = 1024;
constexpr int SNT = 1024;

// Inner tiles an item visits. Query-tile items (forward, dQ) visit key tiles
// [first, last): all of them, or up to the causal limit, and with a sliding window of W keys
// from the tile holding key t*ti - W + 1 (win_first_ktile); key-tile items (dK/dV) visit query
// tiles from the causal start to the last query whose window reaches the item's last key. Item
// ranges [lo, hi) count from the first visited tile.
__device__ __forceinline__ int item_cost(int mode, int causal, int win, int Lq, int Lk, int t,
                                         int ti, int tl) {
  if (mode == SCHED_QTILES) {
    if (Lk <= 0) return 0;
    int nk = (Lk + tl - 1) / tl;
    if (causal) {
      int i_max = min(Lq, (t + 1) * ti) - 1;
      nk = min(nk, i_max / tl + 1);
    }
    return max(0, nk - win_first_ktile(t * ti, win, tl));
  }
  if (Lq <= 0) return 0;
  int nq = (Lq + tl - 1) / tl;
  const int j0 = t * ti;
  int first = 0;
  if (causal) {
    if (j0 >= Lq) return 0;
    first = j0 / tl;
  }
  nq = win_end_qtile(min(Lk, (t + 1) * ti) - 1, win, tl, nq);
  return max(0, nq - first);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// In-place inclusive scan of SNT ints in LDS (all threads participate): a scan inside each wave,
// then a scan of the 16 wave totals by wave 0.
__device__ __forceinline__ void block_scan(int* buf, int* wsum, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  __syncthreads();
  int x = wave_incl_scan(buf[tid], lane);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    const int v = wave_incl_scan(lane < SNT / 64 ? wsum[lane] : 0, lane);
    if (lane < SNT / 64) wsum[lane] = v;
  }
  __syncthreads();
  buf[tid] = x + (w > 0 ? wsum[w - 1] : 0);
  __syncthreads();
}

__global__ __launch_bounds__(SNT) void sched_kernel(SchedArgs a0, SchedArgs a1) {
  const SchedArgs& a = blockIdx.x == 0 ? a0 : a1;
  __shared__ int bucket[NBUCKET];
  __shared__ int cnt[SNT];  // inclusive scan of the chunk's per-sample tile counts
  __shared__ int wsum[SNT / 64];
  __shared__ int err, carry, split_count, slot_count;
  __shared__ unsigned long long wtot[SNT / 64];
  __shared__ int wmax[SNT / 64];
  const int tid = threadIdx.x;
  WsHeader* hdr = (WsHeader*)a.ws_header;
  Item* items = (Item*)a.items;
  for (int i = tid; i < NBUCKET; i += SNT) bucket[i] = 0;
  if (tid == 0) err = 0;
  __syncthreads();
  for (int b = tid; b < a.B; b += SNT) {
    if (a.q_off[b + 1] < a.q_off[b]) atomicOr(&err, 1);
    if (a.q_rows > 0 && a.q_off[b + 1] - a.q_off[b] > a.q_rows) atomicOr(&err, 1);
    if (a.kv_off[b + 1] < a.kv_off[b]) atomicOr(&err, 2);
  }
  if (tid == 0) {
    if (a.q_off[0] != 0 || (int64_t)a.q_off[a.B] != a.total_q) atomicOr(&err, 1);
    if (a.kv_off[0] != 0 || (int64_t)a.kv_off[a.B] != a.total_kv) atomicOr(&err, 2);
  }
  __syncthreads();
  if (err != 0) {
    if (tid == 0) {
      hdr->error = err;
      if (a.list == 0) {
        hdr->n_items = 0; hdr->n_split = 0;
      } else {
        hdr->n_items2 = 0; hdr->n_split2 = 0;
      }
    }
    return;
  }
  const int ti = a.tile_item, tl = a.tile_loop;
  auto ntiles = [&](int b) {
    const int Lq = a.q_off[b + 1] - a.q_off[b];
    const int Lk = a.kv_off[b + 1] - a.kv_off[b];
    return a.mode == SCHED_QTILES ? (Lq + ti - 1) / ti : (Lk + ti - 1) / ti;
  };
  // Walk the samples chunk by chunk; for every tile of the chunk call f(b, t, canonical index).
  auto for_each_tile = [&](auto&& f) {
    if (tid == 0) carry = 0;
    for (int base = 0; base < a.B; base += SNT) {
      const int b = base + tid;
      const int n = b < a.B ? ntiles(b) : 0;
      __syncthreads();
      cnt[tid] = n;
      block_scan(cnt, wsum, tid);
      const int total = cnt[SNT - 1];
      const int first = carry;
      for (int u = tid; u < total; u += SNT) {
        // sample of tile u: first index k with cnt[k] > u
        int lo = 0, hi = SNT - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (cnt[mid] > u) hi = mid; else lo = mid + 1;
        }
        const int t = u - (lo > 0 ? cnt[lo - 1] : 0);
        f(base + lo, t, first + u);
      }
      if (a.tile_base != nullptr && b < a.B) a.tile_base[b] = first + cnt[tid] - n;
      __syncthreads();
      if (tid == 0) carry = first + total;
      __syncthreads();
    }
  };
  // 1. histogram of tile costs (bucket NBUCKET-1-cost puts expensive items first), and with
  //    splitting the total cost (all heads) and the largest tile cost, reduced over the block
  unsigned long long tot = 0;
  int mx = 0;
  for_each_tile([&](int b, int t, int) {
    const int Lq = a.q_off[b + 1] - a.q_off[b];
    const int Lk = a.kv_off[b + 1] - a.kv_off[b];
    const int c = item_cost(a.mode, a.causal, a.win, Lq, Lk, t, ti, tl);
    atomicAdd(&bucket[NBUCKET - 1 - min(c, NBUCKET - 1)], a.H);
    tot += (unsigned long long)c;
    mx = max(mx, c);
  });
  int T = 0x7fffffff;  // chunk length; no splitting unless a tile costs more
  if (a.split) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      tot += __shfl_xor(tot, off, 64);
      mx = max(mx, __shfl_xor(mx, off, 64));
    }
    if ((tid & 63) == 0) {
      wtot[tid >> 6] = tot;
      wmax[tid >> 6] = mx;
    }
    __syncthreads();
    unsigned long long total = 0;
    int biggest = 0;
    for (int w = 0; w < SNT / 64; ++w) {
      total += wtot[w];
      biggest = max(biggest, wmax[w]);
    }
    total *= (unsigned long long)a.H;
    const unsigned long long tpc = (total + a.nslot - 1) / a.nslot;
    const int t_mean = (int)min(max(tpc, (unsigned long long)SPLIT_MIN_TILES), (unsigned long long)0x7fffffff);
    if (biggest > t_mean) {
      T = t_mean;
      // some tiles are split: the histogram counts chunks instead
      __syncthreads();
      bucket[tid] = 0;
      __syncthreads();
      for_each_tile([&](int b, int t, int) {
        const int Lq = a.q_off[b + 1] - a.q_off[b];
        const int Lk = a.kv_off[b + 1] - a.kv_off[b];
        const int c = item_cost(a.mode, a.causal, a.win, Lq, Lk, t, ti, tl);
        const int n = c > T ? (c + T - 1) / T : 1;
        for (int k = 0; k < n; ++k) {
          const int cc = n == 1 ? c : min(T, c - k * T);
          atomicAdd(&bucket[NBUCKET - 1 - min(cc, NBUCKET - 1)], a.H);
        }
      });
    }
  }
  if (tid == 0) {
    split_count = 0;
    slot_count = 0;
  }
  // chunks of a tile of cost c: ceil(c / T) when c > T (the last one may be shorter), else one
  auto chunks = [&](int c) { return c > T ? (c + T - 1) / T : 1; };
  __syncthreads();
  // 2. exclusive scan over the buckets (NBUCKET == SNT)
  const int own = bucket[tid];
  block_scan(bucket, wsum, tid);
  const int total_items = bucket[NBUCKET - 1];
  __syncthreads();
  bucket[tid] -= own;
  __syncthreads();
  // 3. scatter the chunks (b, tile, h, canonical tile index, inner range, slot, chunk); a split
  //    tile takes n consecutive slots per head, and its counter (at the first slot) is cleared
  for_each_tile([&](int b, int t, int canon) {
    const int Lq = a.q_off[b + 1] - a.q_off[b];
    const int Lk = a.kv_off[b + 1] - a.kv_off[b];
    const int c = item_cost(a.mode, a.causal, a.win, Lq, Lk, t, ti, tl);
    const int n = chunks(c);
    int sbase = -1;
    if (n > 1) {
      sbase = atomicAdd(&slot_count, n * a.H);
      atomicAdd(&split_count, a.H);
      if (sbase + n * a.H > 2 * a.nslot) {
        atomicOr(&err, 4);  // cannot happen: the chunk length bounds the slot count
        sbase = -1;
      } else {
        for (int h = 0; h < a.H; ++h) a.split_cnt[sbase + h * n] = 0;  // chunks done per tile
      }
    }
    if (a.split_slot != nullptr)
      for (int h = 0; h < a.H; ++h) a.split_slot[(int64_t)canon * a.H + h] = sbase < 0 ? -1 : sbase + h * n;
    for (int k = 0; k < n; ++k) {
      const int cc = n == 1 ? c : min(T, c - k * T);
      const int pos = atomicAdd(&bucket[NBUCKET - 1 - min(cc, NBUCKET - 1)], a.H);
      for (int h = 0; h < a.H; ++h) {
        if (pos + h < a.max_items) {
          Item it;
          it.b = b; it.tile = t; it.h = h; it.aux = canon;
          it.lo = n == 1 ? 0 : k * T;
          it.hi = n == 1 ? c : min(c, (k + 1) * T);
          it.slot = sbase < 0 ? -1 : sbase + h * n + k;
          it.chunk = sbase < 0 ? 0 : k | (n << 16);
          items[pos + h] = it;
        }
      }
    }
  });
  __syncthreads();
  if (tid == 0) {
    // Only the first list writes the error word (both lists see the same offsets); a list that
    // failed on its own is left empty.
    if (a.tile_base != nullptr) a.tile_base[a.B] = carry;
    const int n = err != 0 ? 0 : min(total_items, a.max_items);
    const int ns = err != 0 ? 0 : split_count;
    const int chunk = a.split && T != 0x7fffffff ? T : 0;
    if (a.list == 0) {
      hdr->error = err;
      hdr->n_items = n; hdr->n_split = ns; hdr->chunk = chunk;
    } else {
      hdr->n_items2 = n; hdr->n_split2 = ns; hdr->chunk2 = chunk;
    }
  }
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t s) {
  prof_before(PROF_SCHED, s);
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(SNT), 0, s, a, a);
  prof_after(PROF_SCHED, s);
  return hipGetLastError();
}

hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t s) {
  prof_before(PROF_SCHED, s);
  hipLaunchKernelGGL(sched_kernel, dim3(2), dim3(SNT), 0, s, a, b);
  prof_after(PROF_SCHED, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Bias gradient, stage A: one thread per (sample, head, diagonal c) sums the partial rows of the
// sample's 32-query row blocks in block order. Row block rb of sample b (queries 32rb..32rb+31)
// is stored at canonical row (tile_base[b] + rb / R) * R + rb % R, R = row blocks per dQ item,
// and wrote exactly the clamped
// diagonals of its raw range [32rb - (k_end - 1), 32rb + 31], k_end = keys it visited; the edge
// entries 0 and NB-1 collect every raw diagonal that clamps to them.
// Inner tiles a dQ item of query tile t visits: key tiles [first, first + count) (all key tiles,
// or those up to the causal limit, from the first one its sliding window reaches).
template <int QI, int KL>
__device__ __forceinline__ int qtile_cost(int t, int Lq, int Lk, int causal, int win, int& first) {
  first = win_first_ktile(t * QI, win, KL);
  if (Lk <= 0) return 0;
  int nkt = (Lk + KL - 1) / KL;
  if (causal) nkt = min(nkt, (min(Lq, (t + 1) * QI) - 1) / KL + 1);
  return max(0, nkt - first);
}

// Raw diagonal range [d_lo, d_hi] that row block rb wrote while its item (or chunk) visited key
// tiles [lo, hi): the wave starts at the first tile its window reaches and stops after its
// causal limit; false if it visited none.
template <int KL>
__device__ __forceinline__ bool chunk_range(int rb, int Lq, int causal, int win, int lo, int hi,
                                            int& d_lo, int& d_hi) {
  const int wrow = rb * 32;
  if (wrow >= Lq) return false;
  int last = hi - 1;
  if (causal) last = min(last, (wrow + 31) / KL);  // tiles after the block's last query skipped
  lo = max(lo, win_first_ktile(wrow, win, KL));    // tiles before its window skipped
  if (lo > last) return false;
  d_lo = wrow - (last + 1) * KL + 1;
  d_hi = wrow + 31 - lo * KL;
  return true;
}

// Loads are issued in batches of 8 row blocks before any of them is added, so a thread waits on
// one memory round trip per batch rather than per row block. A row block whose range misses
// entry c contributes +0.0, which leaves the running sum unchanged: the summation order, and so
// the result bits, are those of the plain loop over rb.
// The tile sizes are template parameters so that the per-row-block range arithmetic divides by
// constants.
template <int QI, int KL, bool WIN>
__global__ __launch_bounds__(256) void dbias_stage_a(DbiasArgs a) {
  const int win = WIN ? a.win : 0;  // a compile-time zero without a window
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= a.nb) return;
  const WsHeader* hdr = (const WsHeader*)a.hdr;
  float acc = 0.0f;
  if (hdr->error == 0) {
    const int Lq = a.q_off[b + 1] - a.q_off[b];
    const int Lk = a.kv_off[b + 1] - a.kv_off[b];
    const int nrb = (Lq + 31) / 32;
    const int tb = a.tile_base[b];
    const int nb = a.nb;
    constexpr int PER = QI / 32;
    constexpr int BATCH = 16;
    // Row block rb reaches diagonals up to 32 rb + 31 (clamped), so entry c sees only row blocks
    // rb >= (c - 31) / 32: the loop starts at the wave's first such block (its lowest c) and is
    // empty past the last row block. Blocks it skips would each have added +0.0. The range
    // arithmetic is uniform across the wave; every lane loads its entry of the row (in bounds,
    // and the wave's 64 entries overlap the row's range anyway) and keeps it only inside the
    // range, so the loads carry no branches.
    const int c_first = __builtin_amdgcn_readfirstlane(c);
    // With a sliding window a row block's first visited key tile starts at most KL - 1 keys
    // before its first query's window, so it wrote no diagonal above win + KL + 29: a wave whose
    // entries all lie above that sums nothing.
    const bool above_window = WIN && c_first > win + KL + 29;
    const int rb_begin = c_first > 32 * nrb - 1 || above_window ? nrb : max(0, (c_first - 31) / 32);
    if (a.split_slot == nullptr || hdr->n_split == 0) {
      // no split tiles: one row per row block. All loads of a batch first (in bounds, no
      // branches), then the range tests; an entry outside its row block's range is cleared by a
      // bit mask (stale bits there may be anything, even NaN), which also keeps every load used.
      for (int rb0 = rb_begin; rb0 < nrb; rb0 += BATCH) {
        int xi[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int rb = min(rb0 + u, nrb - 1);
          const int64_t row = (int64_t)(tb + rb / PER) * PER + rb % PER;
          xi[u] = __float_as_int(a.part[(row * a.H + h) * nb + c]);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int rb = min(rb0 + u, nrb - 1);
          int kf;
          const int nkt = qtile_cost<QI, KL>(rb / PER, Lq, Lk, a.causal, win, kf);
          int d_lo = 1, d_hi = 0;
          const bool any = rb0 + u < nrb && chunk_range<KL>(rb, Lq, a.causal, win, kf, kf + nkt, d_lo, d_hi);
          const bool keep = any && c >= clampi(d_lo, 0, nb - 1) && c <= clampi(d_hi, 0, nb - 1);
          acc += __int_as_float(xi[u] & (keep ? -1 : 0));
        }
      }
    } else for (int rb0 = rb_begin; rb0 < nrb; rb0 += BATCH) {
      float v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int rb = min(rb0 + u, nrb - 1);
        const int t = rb / PER;
        int kf;
        const int nkt = qtile_cost<QI, KL>(t, Lq, Lk, a.causal, win, kf);
        const int sb = a.split_slot[(int64_t)(tb + t) * a.H + h];
        int d_lo = 1, d_hi = 0;
        const bool any = rb0 + u < nrb && sb < 0 && chunk_range<KL>(rb, Lq, a.causal, win, kf, kf + nkt, d_lo, d_hi);
        const int64_t row = (int64_t)(tb + t) * PER + rb % PER;
        const float x = a.part[(row * a.H + h) * nb + c];
        v[u] = any && c >= clampi(d_lo, 0, nb - 1) && c <= clampi(d_hi, 0, nb - 1) ? x : 0.0f;
        if (sb >= 0 && rb0 + u < nrb) {
          // split tile: its chunks' rows, in chunk order
          const int T = hdr->chunk;
          const int n = (nkt + T - 1) / T;
          float sv = 0.0f;
          for (int k = 0; k < n; ++k) {
            if (chunk_range<KL>(rb, Lq, a.causal, win, kf + k * T, kf + min(nkt, (k + 1) * T), d_lo, d_hi) &&
                c >= clampi(d_lo, 0, nb - 1) && c <= clampi(d_hi, 0, nb - 1))
              sv += a.part_x[((int64_t)(sb + k) * PER + rb % PER) * nb + c];
          }
          v[u] = sv;
        }
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) acc += v[u];
    }
  }
  a.part_bh[((int64_t)b * a.H + h) * a.nb + c] = acc;
}

// Stage B: dbias[h, c] = sum over samples in order (loads batched as in stage A).
__global__ __launch_bounds__(256) void dbias_stage_b(DbiasArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.H * a.nb) return;
  const int64_t stride = (int64_t)a.H * a.nb;
  constexpr int BATCH = 16;
  float acc = 0.0f;
  for (int b0 = 0; b0 < a.B; b0 += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[u] = b0 + u < a.B ? a.part_bh[(b0 + u) * stride + idx] : 0.0f;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) acc += v[u];
  }
  a.dbias[idx] = acc;
}

hipError_t launch_dbias_reduce(const DbiasArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.H * a.nb;
  if (n <= 0) return hipSuccess;
  if (a.B > 0) {
    const dim3 grid(a.B * a.H, (a.nb + 255) / 256);
    if (a.tile_rows == 128 && a.loop_rows == 64) {
      if (a.win > 0) hipLaunchKernelGGL((dbias_stage_a<128, 64, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((dbias_stage_a<128, 64, false>), grid, dim3(256), 0, s, a);
    } else if (a.tile_rows == 64 && a.loop_rows == 64) {
      hipLaunchKernelGGL((dbias_stage_a<64, 64, false>), grid, dim3(256), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dbias_stage_b, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Shared query block: dQ[i, h, :] = the sum of the samples' fp32 gradient rows for query i. A
// workgroup owns one (i, h); each thread holds 4 columns of a row and takes the samples s,
// s + S, s + 2S, ... (S = 256 / (D / 4) rows in flight), then one thread per 4 columns adds
// the S partial sums in order. The order is fixed, so the result is bitwise reproducible; it is
// rounded once to bf16, or written in fp32 for fp32 problems. Only
// 256 workgroups run for the PMA shape, so a thread issues the offsets of U samples, then their
// U row loads, before it adds anything: two memory latencies per U samples.
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void dq_shared_reduce(DqSharedArgs a) {
  constexpr int LPR = D / 4, S = 256 / LPR, U = 16;
  __shared__ f32x4 red[256];
  const WsHeader* hdr = (const WsHeader*)a.hdr;
  if (hdr->error != 0) return;
  const int i = blockIdx.x / a.H, h = blockIdx.x - i * a.H;
  const int tid = threadIdx.x, c = tid % LPR, s = tid / LPR;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int b0 = s; b0 < a.B; b0 += U * S) {
    int q0[U], q1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * S, a.B - 1);
      q0[u] = a.q_off[b];
      q1[u] = a.q_off[b + 1];
    }
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (b0 + u * S < a.B && i < q1[u] - q0[u])
        v[u] = *(const f32x4*)(a.part + ((int64_t)(q0[u] + i) * a.H + h) * D + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u];
  }
  red[tid] = acc;
  __syncthreads();
  if (tid < LPR) {
    f32x4 t = red[c];
    for (int k = 1; k < S; ++k) t += red[k * LPR + c];
    if (F32OUT) {
      *(f32x4*)((float*)a.dQ + ((int64_t)i * a.H + h) * D + 4 * c) = t;
    } else {
      const bf16x2 lo = pack_bf16(t[0], t[1]), hi = pack_bf16(t[2], t[3]);
      *(bf16x4*)((__bf16*)a.dQ + ((int64_t)i * a.H + h) * D + 4 * c) = bf16x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
}

hipError_t launch_dq_shared_reduce(const DqSharedArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.q_rows * a.H;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n);
  if (a.f32_out) {
    if (a.D == 32) hipLaunchKernelGGL((dq_shared_reduce<32, true>), grid, dim3(256), 0, s, a);
    else if (a.D == 64) hipLaunchKernelGGL((dq_shared_reduce<64, true>), grid, dim3(256), 0, s, a);
    else if (a.D == 128) hipLaunchKernelGGL((dq_shared_reduce<128, true>), grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.D == 32) hipLaunchKernelGGL((dq_shared_reduce<32, false>), grid, dim3(256), 0, s, a);
    else if (a.D == 64) hipLaunchKernelGGL((dq_shared_reduce<64, false>), grid, dim3(256), 0, s, a);
    else if (a.D == 128) hipLaunchKernelGGL((dq_shared_reduce<128, false>), grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdpa
