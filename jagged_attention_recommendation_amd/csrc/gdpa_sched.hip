// Jagged work scheduler.
//
// Short sequences must not leave compute units idle while long ones finish (page "GEM Training:
// How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", JFA paragraph; the GDPA
// paragraph adds that short or asymmetric K/V and large batches break occupancy assumptions and
// that scheduling was redesigned). This kernel turns the offsets into a list of equal-shaped work
// items, one per (sample, head, tile), sorted by decreasing cost: the cost of an item is the
// number of inner-loop tiles it visits (all key tiles, or only those with j <= i under causal
// masking). Workgroups are handed out by the hardware in index order, so the longest items start
// first and short ones fill the gaps at the end (longest-processing-time-first list scheduling).
//
// One workgroup of 1024 threads: validate offsets, histogram costs, scan, scatter. The relative
// order of equal-cost items is not fixed, which cannot change results: every item computes its
// outputs on its own.
#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

constexpr int NBUCKET = 1024;

__device__ __forceinline__ int item_cost(int mode, int causal, int Lq, int Lk, int t, int ti,
                                         int tl) {
  if (mode == SCHED_QTILES) {
    if (Lk <= 0) return 0;
    int nk = (Lk + tl - 1) / tl;
    if (!causal) return nk;
    int i_max = min(Lq, (t + 1) * ti) - 1;
    return min(nk, i_max / tl + 1);
  }
  if (Lq <= 0) return 0;
  int nq = (Lq + tl - 1) / tl;
  if (!causal) return nq;
  int j0 = t * ti;
  if (j0 >= Lq) return 0;
  return nq - j0 / tl;
}

__global__ __launch_bounds__(1024) void sched_kernel(SchedArgs a) {
  __shared__ int bucket[NBUCKET];
  __shared__ int err;
  const int tid = threadIdx.x;
  WsHeader* hdr = (WsHeader*)a.ws_header;
  Item* items = (Item*)a.items;
  for (int i = tid; i < NBUCKET; i += blockDim.x) bucket[i] = 0;
  if (tid == 0) err = 0;
  __syncthreads();
  for (int b = tid; b < a.B; b += blockDim.x) {
    if (a.q_off[b + 1] < a.q_off[b]) atomicOr(&err, 1);
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
      if (a.list == 0) hdr->n_items = 0; else hdr->n_items2 = 0;
    }
    return;
  }
  const int ti = a.tile_item, tl = a.tile_loop;
  // 1. histogram of costs; bucket index NBUCKET-1-cost puts expensive items first
  for (int b = tid; b < a.B; b += blockDim.x) {
    int Lq = a.q_off[b + 1] - a.q_off[b];
    int Lk = a.kv_off[b + 1] - a.kv_off[b];
    int n = a.mode == SCHED_QTILES ? (Lq + ti - 1) / ti : (Lk + ti - 1) / ti;
    for (int t = 0; t < n; ++t) {
      int c = min(item_cost(a.mode, a.causal, Lq, Lk, t, ti, tl), NBUCKET - 1);
      atomicAdd(&bucket[NBUCKET - 1 - c], a.H);
    }
  }
  __syncthreads();
  // 2. exclusive scan over the buckets (NBUCKET == blockDim.x)
  int own = bucket[tid];
  for (int off = 1; off < NBUCKET; off <<= 1) {
    __syncthreads();
    int add = tid >= off ? bucket[tid - off] : 0;
    __syncthreads();
    bucket[tid] += add;
  }
  __syncthreads();
  int total = bucket[NBUCKET - 1];
  __syncthreads();
  bucket[tid] -= own;
  __syncthreads();
  // 3. scatter (b, tile, h) records. Samples are walked in chunks of blockDim.x; a scan of the
  //    per-sample tile counts gives each sample's canonical first-tile index (tile_base), which
  //    items carry in .aux.
  __shared__ int cnt[NBUCKET];
  __shared__ int carry;
  if (tid == 0) carry = 0;
  for (int base = 0; base < a.B; base += blockDim.x) {
    const int b = base + tid;
    int Lq = 0, Lk = 0, n = 0;
    if (b < a.B) {
      Lq = a.q_off[b + 1] - a.q_off[b];
      Lk = a.kv_off[b + 1] - a.kv_off[b];
      n = a.mode == SCHED_QTILES ? (Lq + ti - 1) / ti : (Lk + ti - 1) / ti;
    }
    __syncthreads();
    cnt[tid] = n;
    for (int off = 1; off < NBUCKET; off <<= 1) {
      __syncthreads();
      int add = tid >= off ? cnt[tid - off] : 0;
      __syncthreads();
      cnt[tid] += add;
    }
    __syncthreads();
    const int first = carry + cnt[tid] - n;
    if (b < a.B) {
      if (a.tile_base != nullptr) a.tile_base[b] = first;
      for (int t = 0; t < n; ++t) {
        int cost = item_cost(a.mode, a.causal, Lq, Lk, t, ti, tl);
        int c = min(cost, NBUCKET - 1);
        int pos = atomicAdd(&bucket[NBUCKET - 1 - c], a.H);
        for (int h = 0; h < a.H; ++h) {
          if (pos + h < a.max_items) {
            Item it;
            it.b = b; it.tile = t; it.h = h; it.aux = first + t;
            items[pos + h] = it;
          }
        }
      }
    }
    __syncthreads();
    if (tid == blockDim.x - 1) carry += cnt[tid];
  }
  __syncthreads();
  if (tid == 0) {
    if (a.tile_base != nullptr) a.tile_base[a.B] = carry;
    hdr->error = 0;
    int n = min(total, a.max_items);
    if (a.list == 0) hdr->n_items = n; else hdr->n_items2 = n;
  }
}

// One thread per (h, r): walks samples and their query tiles in canonical order and adds every
// partial row entry that tile wrote for diagonal r.
__global__ __launch_bounds__(256) void dbias_reduce_kernel(DbiasArgs a) {
  const WsHeader* hdr = (const WsHeader*)a.hdr;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.H * a.nb) return;
  const int h = (int)(idx / a.nb), r = (int)(idx % a.nb);
  float acc = 0.0f;
  if (hdr->error == 0) {
    const int TMr = a.tile_rows, nb = a.nb;
    for (int b = 0; b < a.B; ++b) {
      const int Lq = a.q_off[b + 1] - a.q_off[b];
      const int Lk = a.kv_off[b + 1] - a.kv_off[b];
      if (Lk <= 0) continue;
      const int nt = (Lq + TMr - 1) / TMr;
      const int tb = a.tile_base[b];
      for (int t = 0; t < nt; ++t) {
        const int i0 = t * TMr;
        const int c_lo = clampi(i0 - (Lk - 1), 0, nb - 1);
        const int c_hi = clampi(min(Lq, i0 + TMr) - 1, 0, nb - 1);
        if (r >= c_lo && r <= c_hi) acc += a.part[((int64_t)(tb + t) * a.H + h) * nb + r];
      }
    }
  }
  a.dbias[idx] = acc;
}

hipError_t launch_dbias_reduce(const DbiasArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.H * a.nb;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t s) {
  prof_before(PROF_SCHED, s);
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(NBUCKET), 0, s, a);
  prof_after(PROF_SCHED, s);
  return hipGetLastError();
}

}  // namespace gdpa
