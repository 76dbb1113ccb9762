// Jagged work scheduler and the bias-gradient reduction.
//
// Short sequences must not leave compute units idle while long ones finish (page "GEM Training:
// How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", JFA paragraph; the GDPA
// paragraph adds that short or asymmetric K/V and large batches break occupancy assumptions and
// that scheduling was redesigned). The scheduler turns the offsets into a list of equal-shaped
// work items, one per (sample, head, tile) or per chunk of a long tile. The cost of an item is
// the number of inner-loop tiles it visits (all tiles, or only those allowed by causal masking
// and the sliding window).
//
// Placement. The GPU has eight accelerator dies, each with its own L2 cache; the dispatcher
// hands workgroup i to die i % 8, and each die consumes its own workgroups in index order. The
// items of one (sample, head) group all read the same K and V (query tiles) or Q and dO (key
// tiles), so a group is kept on one die: groups are ranked by cost, largest first, and dealt to
// the dies in a snake (0..7, 7..0, ...), which balances the dies' total cost. On each die the
// groups run in rank order with a group's items consecutive (costliest tile first), so a group's
// items start together and stream the shared operand through that die's L2 in step, and the
// cheapest groups fill the end. Die x's q-th item goes to list index 8q + x; when the dies hold
// different item counts, the surplus at the end of a longer die's sequence fills the missing
// indices of the shorter ones, so the list stays dense. Equal-cost groups are ranked in no fixed
// order, which cannot change results: every item computes its outputs on its own, and split
// tiles combine their chunks in chunk order.
//
// One workgroup of 1024 threads per list (the backward builds its query-tile and key-tile lists
// in one launch). Samples are walked in chunks of 1024, a scan of their tile counts gives each
// tile a canonical index, and threads then take tiles (not samples) so long samples do not
// serialise. Per-sample values live in LDS when the batch fits one chunk, else in workspace
// scratch. A long list whose tiles all fit one item is written by a second launch of one thread
// per tile over many workgroups, from the ranks and positions the list's workgroup leaves in the
// workspace.
#include <atomic>

#include "gdpa_common.h"
#include "gdpa_internal.h"

namespace gdpa {

constexpr int NBUCKET = 1024;
constexpr int SNT = 1024;
constexpr int XCDS = 8;      // accelerator dies
constexpr int GCAP = 4096;   // (sample, head) groups whose placement table fits in LDS
constexpr int OCAP = 16384;  // tiles of a chunk of samples whose owning sample is looked up in LDS

// Inner tiles an item visits. Query-tile items (forward, dQ) visit key tiles
// [first, last): all of them, or up to the causal limit, and with a sliding window of W keys
// from the tile holding key t*ti - W + 1; key-tile items (dK/dV) visit query tiles from the
// causal start to the last query whose window reaches the item's last key. Item ranges [lo, hi)
// count from the first visited tile. Tile sizes are powers of two, passed as shifts (tis, tls);
// every quotient below has a non-negative dividend.
__device__ __forceinline__ int item_cost(int mode, int causal, int win, int Lq, int Lk, int t,
                                         int tis, int tls) {
  const int tl = 1 << tls;
  if (mode == SCHED_QTILES) {
    if (Lk <= 0) return 0;
    int nk = (Lk + tl - 1) >> tls;
    const int q_lo = t << tis;
    if (causal) nk = min(nk, ((min(Lq, q_lo + (1 << tis)) - 1) >> tls) + 1);
    const int first = win > 0 ? max(0, q_lo - win + 1) >> tls : 0;
    return max(0, nk - first);
  }
  if (Lq <= 0) return 0;
  int nq = (Lq + tl - 1) >> tls;
  const int j0 = t << tis;
  int first = 0;
  if (causal) {
    if (j0 >= Lq) return 0;
    first = j0 >> tls;
  }
  if (win > 0) nq = min(nq, ((min(Lk, j0 + (1 << tis)) - 1 + win - 1) >> tls) + 1);
  return max(0, nq - first);
}

// Rank bucket of a group cost, larger costs first: exact below 512, then eight buckets per
// octave.
__device__ __forceinline__ int cost_bucket(unsigned long long c) {
  int key;
  if (c < 512) {
    key = (int)c;
  } else {
    const int o = 63 - __clzll(c);  // 9 .. 63
    key = min(NBUCKET - 1, 512 + (o - 9) * 8 + (int)((c >> (o - 3)) & 7));
  }
  return NBUCKET - 1 - key;
}

// Die of group rank r (snake over the dies) and its rank among that die's groups.
__device__ __forceinline__ int group_xcd(int r) {
  const int s = r & 15;
  return s < XCDS ? s : 2 * XCDS - 1 - s;
}

// List index of die x's q-th item. The dies' own counts are xtot; tgt[x] = indices below the list
// length n that are x mod 8; a die with more items than that passes its surplus on, spre and dpre
// being the prefix sums of surplus and shortfall over the dies (dpre[8] = total shortfall).
__device__ __forceinline__ int list_position(const int* xtot, const int* tgt, const int* spre,
                                             const int* dpre, int x, int q) {
  if (q < tgt[x]) return XCDS * q + x;
  const int k = spre[x] + (q - tgt[x]);  // surplus item k fills the k-th missing index
  int y = 0;
  while (y < XCDS - 1 && k >= dpre[y + 1]) ++y;
  return XCDS * (xtot[y] + k - dpre[y]) + y;
}

// tgt, spre and dpre of list_position from the dies' own counts (one thread).
__device__ __forceinline__ void die_tables(const int* xtot, int* tgt, int* spre, int* dpre) {
  int n = 0;
  for (int x = 0; x < XCDS; ++x) n += xtot[x];
  int sp = 0, dp = 0;
  for (int x = 0; x < XCDS; ++x) {
    tgt[x] = n / XCDS + (x < n % XCDS ? 1 : 0);  // indices x, x + 8, ... below n
    spre[x] = sp;
    dpre[x] = dp;
    sp += max(0, xtot[x] - tgt[x]);
    dp += max(0, tgt[x] - xtot[x]);
  }
  dpre[XCDS] = dp;
}

// Inclusive scan over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4 and 8 within
// each row of 16 lanes, then row 0's total into row 1, row 2's into row 3, and lane 31's running
// total into rows 2 and 3. A lane whose source falls outside its row adds zero.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Sum and maximum over the 64 lanes of a wave, returned to lane 63, with the moves of
// wave_incl_scan (64-bit sum carried as two 32-bit halves).
template <int CTRL, int RMASK>
__device__ __forceinline__ void sum_max_step(unsigned long long& s, int& m) {
  const unsigned lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)s, CTRL, RMASK, 0xf, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(s >> 32), CTRL, RMASK, 0xf, false);
  s += ((unsigned long long)hi << 32) | lo;
  m = max(m, __builtin_amdgcn_update_dpp(0, m, CTRL, RMASK, 0xf, false));
}
__device__ __forceinline__ void wave_sum_max(unsigned long long& s, int& m) {
  sum_max_step<0x111, 0xf>(s, m);
  sum_max_step<0x112, 0xf>(s, m);
  sum_max_step<0x114, 0xf>(s, m);
  sum_max_step<0x118, 0xf>(s, m);
  sum_max_step<0x142, 0xa>(s, m);
  sum_max_step<0x143, 0xc>(s, m);
}

// In-place inclusive scan of SNT ints in LDS (all threads participate): a scan inside each wave,
// then a scan of the 16 wave totals by wave 0.
__device__ __forceinline__ void block_scan(int* buf, int* wsum, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  __syncthreads();
  int x = wave_incl_scan(buf[tid]);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    const int v = wave_incl_scan(lane < SNT / 64 ? wsum[lane] : 0);
    if (lane < SNT / 64) wsum[lane] = v;
  }
  __syncthreads();
  buf[tid] = x + (w > 0 ? wsum[w - 1] : 0);
  __syncthreads();
}

// One list per workgroup: workgroup i builds lists.l[i] (indexed in the kernel-argument segment;
// choosing among separate arguments made the compiler copy them to scratch memory).
struct SchedLists {
  SchedArgs l[3];
};

// SMALL: the batch fits one chunk of samples and its groups fit the LDS placement table, so every
// per-sample and per-group value lives in LDS; otherwise they go through the workspace scratch.
template <bool SMALL>
__global__ __launch_bounds__(SNT) void sched_kernel(SchedLists lists) {
  const SchedArgs& a = lists.l[blockIdx.x];
  __shared__ int cnt[SNT];   // inclusive scan of the chunk's per-sample tile counts
  __shared__ int sbuf[SNT];  // scan of chunk counts per tile
  __shared__ int wsum[SNT / 64];
  __shared__ int lq_c[SNT], lk_c[SNT];       // lengths of the chunk's samples
  __shared__ int q0_c[SNT], kv0_c[SNT];      // their first query and key rows
  __shared__ unsigned long long ccost[SNT];  // per-sample cost (one head) of the chunk
  __shared__ int cnch[SNT];                  // per-sample item count (one head) of the chunk
  __shared__ int first_e[SNT];               // chunk index of each sample's first tile
  __shared__ int s_rank[SMALL ? SNT : 1], s_at[SMALL ? SNT : 1];  // rank of a sample / its inverse
  __shared__ int s_gpre[SMALL ? GCAP : 1];   // first position of each group on its die
  __shared__ int bucket[NBUCKET];
  __shared__ unsigned short owner[OCAP];  // local sample of each of the chunk's first OCAP tiles
  // one batch of tiles between their numbering and their items: local sample, tile, cost,
  // chunks, first chunk number within the sample, first chunk slot
  __shared__ int bt_bl[SNT], bt_t[SNT], bt_c[SNT], bt_n[SNT], bt_ci[SNT], bt_sb[SNT];
  __shared__ int xtot[XCDS], tgt[XCDS], spre[XCDS], dpre[XCDS + 1];
  __shared__ int err, carry, split_count, slot_count, big_sh, t_sh;
  __shared__ unsigned long long tot_sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  WsHeader* hdr = (WsHeader*)a.ws_header;
  Item* items = (Item*)a.items;
  const int B = a.B, H = a.H, G = B * H;
  // per-sample and per-group tables
  auto cost_of_sample = [&](int b) -> unsigned long long {
    if constexpr (SMALL) return ccost[b]; else return a.scratch_cost[b];
  };
  auto nch_of = [&](int b) -> int {
    if constexpr (SMALL) return cnch[b]; else return a.scratch_nch[b];
  };
  auto rank_of = [&](int b) -> int {
    if constexpr (SMALL) return s_rank[b]; else return a.scratch_rank[b];
  };
  auto sample_at = [&](int r) -> int {
    if constexpr (SMALL) return s_at[r]; else return a.scratch_at[r];
  };
  auto gpre_of = [&](int r) -> int {
    if constexpr (SMALL) return s_gpre[r]; else return a.scratch_gpre[r];
  };

  const int tis = __builtin_ctz(a.tile_item), tls = __builtin_ctz(a.tile_loop);
  const bool qmode = a.mode == SCHED_QTILES;
  // Load chunk [base, base + SNT) of samples (lengths, tile-count scan); returns its tile count.
  // A sample with a negative length (or more queries than a shared query block holds) sets the
  // error word and counts as empty; the first chunk's load also checks the offsets' ends.
  auto load_chunk = [&](int base) {
    const int b = base + tid;
    int n = 0;
    __syncthreads();
    if (base == 0 && tid == 0) {
      // four independent loads (one round trip, not four in a row while every thread waits)
      const int q_first = a.q_off[0], q_last = a.q_off[B], k_first = a.kv_off[0], k_last = a.kv_off[B];
      int e = 0;
      if (q_first != 0 || (int64_t)q_last != a.total_q) e |= 1;
      if (k_first != 0 || (int64_t)k_last != a.total_kv) e |= 2;
      if (e != 0) atomicOr(&err, e);
    }
    if (b < B) {
      int Lq = a.q_off[b + 1] - a.q_off[b], Lk = a.kv_off[b + 1] - a.kv_off[b];
      const int e = (Lq < 0 || (a.q_rows > 0 && Lq > a.q_rows) ? 1 : 0) | (Lk < 0 ? 2 : 0);
      if (e != 0) {
        atomicOr(&err, e);
        Lq = Lk = 0;
      }
      lq_c[tid] = Lq;
      lk_c[tid] = Lk;
      q0_c[tid] = a.q_off[b];
      kv0_c[tid] = a.kv_off[b];
      n = ((qmode ? Lq : Lk) + (1 << tis) - 1) >> tis;
    }
    cnt[tid] = n;
    block_scan(cnt, wsum, tid);
    for (int u = cnt[tid] - n; u < min(cnt[tid], OCAP); ++u) owner[u] = (unsigned short)tid;
    __syncthreads();
    return cnt[SNT - 1];
  };
  // local sample and tile of the chunk's tile u (samples [0, ns) of the chunk)
  auto locate = [&](int u, int ns, int& bl, int& t) {
    int lo = 0;
    if (u < OCAP) {
      lo = owner[u];
    } else {
      int hi = ns - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cnt[mid] > u) hi = mid; else lo = mid + 1;
      }
    }
    bl = lo;
    t = u - (lo > 0 ? cnt[lo - 1] : 0);
  };
  auto cost_of = [&](int bl, int t) { return item_cost(a.mode, a.causal, a.win, lq_c[bl], lk_c[bl], t, tis, tls); };

  // 1. per-sample cost (one head), total cost and the largest tile cost
  if (tid == 0) {
    err = 0;
    tot_sh = 0;
    big_sh = 0;
  }
  unsigned long long tot = 0;
  int mx = 0;
  for (int base = 0; base < B; base += SNT) {
    const int total = load_chunk(base);
    if (err != 0) break;  // read after the scan's barrier: uniform
    const int ns = min(SNT, B - base);
    ccost[tid] = 0;
    cnch[tid] = tid < ns ? cnt[tid] - (tid > 0 ? cnt[tid - 1] : 0) : 0;  // tiles
    __syncthreads();
    for (int u = tid; u < total; u += SNT) {
      int bl, t;
      locate(u, ns, bl, t);
      const int c = cost_of(bl, t);
      atomicAdd(&ccost[bl], (unsigned long long)c);
      tot += (unsigned long long)c;
      mx = max(mx, c);
    }
    __syncthreads();
    if (!SMALL && tid < ns) {
      a.scratch_cost[base + tid] = ccost[tid];
      a.scratch_nch[base + tid] = cnch[tid];
    }
  }
  __syncthreads();
  if (err != 0) {
    if (tid == 0) {
      hdr->error = err;
      int* die = a.list == 0 ? hdr->die_items : hdr->die_items2;
      int* qc = a.list == 0 ? hdr->qctr : hdr->qctr2;
      for (int x = 0; x < XCDS; ++x) die[x] = qc[x] = 0;
      if (a.list == 0) {
        hdr->n_items = 0; hdr->n_split = 0;
      } else {
        hdr->n_items2 = 0; hdr->n_split2 = 0;
      }
    }
    return;
  }
  int T = 0x7fffffff;  // chunk length; no splitting unless a tile costs more
  if (a.split) {
    wave_sum_max(tot, mx);  // costs are non-negative: the zero fills add and max nothing
    if (lane == 63) {
      atomicAdd(&tot_sh, tot);
      atomicMax(&big_sh, mx);
    }
    __syncthreads();
    if (tid == 0) {
      const unsigned long long total = tot_sh * (unsigned long long)H;
      const unsigned long long tpc =
          total < 0xffffffffull - a.nslot ? (unsigned)(total + a.nslot - 1) / (unsigned)a.nslot
                                          : (total + a.nslot - 1) / a.nslot;
      const int t_mean = (int)min(max(tpc, (unsigned long long)SPLIT_MIN_TILES), (unsigned long long)0x7fffffff);
      t_sh = big_sh > t_mean ? t_mean : 0x7fffffff;
    }
    __syncthreads();
    T = t_sh;
  }
  // chunks of a tile of cost c: ceil(c / T) when c > T (the last one may be shorter), else one
  auto chunks = [&](int c) { return c > T ? (c + T - 1) / T : 1; };
  if (T != 0x7fffffff) {
    // 1b. with split tiles a sample's item count is its chunk count
    for (int base = 0; base < B; base += SNT) {
      const int total = SMALL ? cnt[SNT - 1] : load_chunk(base);
      const int ns = min(SNT, B - base);
      cnch[tid] = 0;
      __syncthreads();
      for (int u = tid; u < total; u += SNT) {
        int bl, t;
        locate(u, ns, bl, t);
        atomicAdd(&cnch[bl], chunks(cost_of(bl, t)));
      }
      __syncthreads();
      if (!SMALL && tid < ns) a.scratch_nch[base + tid] = cnch[tid];
    }
  }
  // 2. rank the samples by cost, largest first (counting sort over cost buckets)
  for (int i = tid; i < NBUCKET; i += SNT) bucket[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += SNT) atomicAdd(&bucket[cost_bucket(cost_of_sample(b))], 1);
  __syncthreads();
  const int own = bucket[tid];
  block_scan(bucket, wsum, tid);  // NBUCKET == SNT
  bucket[tid] -= own;
  __syncthreads();
  for (int b = tid; b < B; b += SNT) {
    const int r = atomicAdd(&bucket[cost_bucket(cost_of_sample(b))], 1);
    if constexpr (SMALL) {
      s_rank[b] = r;
      if (r < B) s_at[r] = b;
    } else {
      a.scratch_rank[b] = r;
      if (r < B) a.scratch_at[r] = b;
    }
  }
  __syncthreads();
  // 3. group r = rank * H + head goes to die group_xcd(r); wave x lays out die x's groups in rank
  //    order: gpre[r] is the group's first position on its die, xtot[x] the die's item count.
  //    Round k of sixteen ranks holds die x's groups 16k + x and 16k + 15 - x, in that order.
  if (wv < XCDS) {
    const int x = wv;
    int run = 0;
    for (int k0 = 0; 16 * k0 < G; k0 += 64) {
      const int k = k0 + lane;
      const int r0 = 16 * k + x, r1 = 16 * k + 2 * XCDS - 1 - x;
      const int n0 = r0 < G ? nch_of(sample_at(r0 / H)) : 0;
      const int n1 = r1 < G ? nch_of(sample_at(r1 / H)) : 0;
      const int incl = wave_incl_scan(n0 + n1);
      const int excl = run + incl - (n0 + n1);
      if constexpr (SMALL) {
        if (r0 < G) s_gpre[r0] = excl;
        if (r1 < G) s_gpre[r1] = excl + n0;
      } else {
        if (r0 < G) a.scratch_gpre[r0] = excl;
        if (r1 < G) a.scratch_gpre[r1] = excl + n0;
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) xtot[x] = run;
  }
  __syncthreads();
  if (tid == 0) {
    die_tables(xtot, tgt, spre, dpre);
    split_count = 0;
    slot_count = 0;
    carry = 0;
  }
  __syncthreads();
  auto position = [&](int x, int q) { return list_position(xtot, tgt, spre, dpre, x, q); };
  if (SMALL && a.defer && T == 0x7fffffff) {
    // 4'. no split tile: sched_items_kernel writes the items from these tables (in LDS here)
    const int total = cnt[SNT - 1];
    if (tid < B) {
      a.scratch_at[tid] = cnt[tid];
      a.scratch_rank[tid] = s_rank[tid];
      a.scratch_nch[tid] = cnch[tid];
      if (a.tile_base != nullptr) a.tile_base[tid] = tid > 0 ? cnt[tid - 1] : 0;
    }
    for (int r = tid; r < G; r += SNT) a.scratch_gpre[r] = s_gpre[r];
    if (a.split_slot != nullptr)
      for (int i = tid; i < total * H; i += SNT) a.split_slot[i] = -1;
    if (tid == 0) carry = total;
  } else {
    // 4. scatter the items (b, tile, h, canonical tile index, inner range, slot, chunk); a split
    //    tile takes n consecutive slots per head, and its counter (at the first slot) is cleared.
    //    Within a sample, chunks are numbered in tile order (sbuf scan); a group lists its
    //    costliest tiles first: the last query tiles (causal), or the first key tiles. Tiles are
    //    numbered in batches of SNT; the batch's items are then written one (tile, head) pair per
    //    thread.
    for (int base = 0; base < B; base += SNT) {
      const int total = SMALL ? cnt[SNT - 1] : load_chunk(base);  // one chunk: still loaded
      const int ns = min(SNT, B - base);
      const int first = carry;
      if (a.tile_base != nullptr && tid < ns) a.tile_base[base + tid] = first + (tid > 0 ? cnt[tid - 1] : 0);
      int run = 0;  // chunks of the chunk's earlier tiles
      for (int u0 = 0; u0 < total; u0 += SNT) {
        const int u = u0 + tid;
        int bl = 0, t = 0, c = 0, n = 0;
        if (u < total) {
          locate(u, ns, bl, t);
          c = cost_of(bl, t);
          n = chunks(c);
        }
        int ci = t;  // chunk number of the tile's first chunk within its sample
        if (T != 0x7fffffff) {
          __syncthreads();
          sbuf[tid] = n;
          block_scan(sbuf, wsum, tid);
          const int e = run + sbuf[tid] - n;  // first chunk of this tile
          if (u < total && t == 0) first_e[bl] = e;
          __syncthreads();
          run += sbuf[SNT - 1];
          ci = e - first_e[bl];
        }
        int sbase = -1;
        if (u < total && n > 1) {
          sbase = atomicAdd(&slot_count, n * H);
          atomicAdd(&split_count, H);
          if (sbase + n * H > 2 * a.nslot) {
            atomicOr(&err, 4);  // cannot happen: the chunk length bounds the slot count
            sbase = -1;
          } else {
            for (int h = 0; h < H; ++h) a.split_cnt[sbase + h * n] = 0;  // chunks done per tile
          }
        }
        if (u < total && a.split_slot != nullptr)
          for (int h = 0; h < H; ++h) a.split_slot[(int64_t)(first + u) * H + h] = sbase < 0 ? -1 : sbase + h * n;
        __syncthreads();  // the previous batch's items are out
        bt_bl[tid] = bl; bt_t[tid] = t; bt_c[tid] = c; bt_n[tid] = n; bt_ci[tid] = ci; bt_sb[tid] = sbase;
        __syncthreads();
        // items of the batch, one (tile, head) pair per thread at a time
        const int nt_b = min(SNT, total - u0);
        for (int pr = tid; pr < nt_b * H; pr += SNT) {
          const int j = pr / H, h = pr - j * H;
          const int bj = bt_bl[j], tj = bt_t[j], cj = bt_c[j], nj = bt_n[j], cij = bt_ci[j], sbj = bt_sb[j];
          const int b = base + bj;
          const int nb = SMALL ? cnch[bj] : nch_of(b);
          const int r = rank_of(b) * H + h;
          const int x = group_xcd(r), g0 = gpre_of(r);
          Item it;
          it.b = b; it.tile = tj; it.h = h; it.aux = first + u0 + j;
          it.q0 = q0_c[bj]; it.lq = lq_c[bj]; it.kv0 = kv0_c[bj]; it.lk = lk_c[bj];
          for (int k = 0; k < nj; ++k) {
            it.lo = nj == 1 ? 0 : k * T;
            it.hi = nj == 1 ? cj : min(cj, (k + 1) * T);
            it.slot = sbj < 0 ? -1 : sbj + h * nj + k;
            it.chunk = sbj < 0 ? 0 : k | (nj << 16);
            const int w = qmode ? nb - 1 - (cij + k) : cij + k;
            const int pos = position(x, g0 + w);
            if (pos >= 0 && pos < a.max_items) items[pos] = it;
          }
        }
      }
      __syncthreads();
      if (tid == 0) carry = first + total;
      __syncthreads();
    }
  }
  if (tid == 0) {
    // Only the first list writes the error word (both lists see the same offsets); a list that
    // failed on its own is left empty.
    if (a.tile_base != nullptr) a.tile_base[B] = carry;
    int n = 0;
    for (int x = 0; x < XCDS; ++x) n += xtot[x];
    n = err != 0 ? 0 : min(n, a.max_items);
    const int ns = err != 0 ? 0 : split_count;
    const int chunk = a.split && T != 0x7fffffff ? T : 0;
    int* die = a.list == 0 ? hdr->die_items : hdr->die_items2;
    int* qc = a.list == 0 ? hdr->qctr : hdr->qctr2;  // claim counters of the persistent kernels
    for (int x = 0; x < XCDS; ++x) {
      die[x] = err != 0 ? 0 : xtot[x];
      qc[x] = 0;
    }
    if (a.list == 0) {
      hdr->error = err;
      hdr->n_items = n; hdr->n_split = ns; hdr->chunk = chunk;
    } else {
      hdr->n_items2 = n; hdr->n_split2 = ns; hdr->chunk2 = chunk;
    }
  }
}

// Items of deferred lists: one thread per canonical tile, writing the tile's items for every
// head where the list kernel would have put them (same item words, same positions). Workgroups
// [first[i], first[i + 1]) serve list i; a list that split tiles, or failed, was written (or
// left empty) by the list kernel, and its workgroups return.
constexpr int ITEM_NT = 256;  // threads (tiles) per workgroup
struct ItemsGrid {
  int first[4];
};

__global__ __launch_bounds__(ITEM_NT) void sched_items_kernel(SchedLists lists, ItemsGrid grid) {
  int li = 0;
  while (li < 2 && (int)blockIdx.x >= grid.first[li + 1]) ++li;
  const SchedArgs& a = lists.l[li];
  const int part = (int)blockIdx.x - grid.first[li];
  __shared__ int tend[SNT];  // inclusive tile end of each sample
  __shared__ int xtot[XCDS], tgt[XCDS], spre[XCDS], dpre[XCDS + 1];
  __shared__ int go;
  const int tid = threadIdx.x;
  const int B = a.B, H = a.H;
  if (tid == 0) {
    const WsHeader* hdr = (const WsHeader*)a.ws_header;
    const int n = a.list == 0 ? hdr->n_items : hdr->n_items2;
    const int chunk = a.list == 0 ? hdr->chunk : hdr->chunk2;
    const int* die = a.list == 0 ? hdr->die_items : hdr->die_items2;
    for (int x = 0; x < XCDS; ++x) xtot[x] = die[x];
    die_tables(xtot, tgt, spre, dpre);
    // (the launch defers only batches whose samples fit tend)
    go = n > 0 && chunk == 0 && B <= SNT && (int64_t)part * ITEM_NT < (int64_t)n;
  }
  for (int i = tid; i < min(B, SNT); i += ITEM_NT) tend[i] = a.scratch_at[i];
  __syncthreads();
  if (!go) return;
  const int u = part * ITEM_NT + tid;
  if (u >= tend[B - 1]) return;
  int b = 0, hi = B - 1;  // first sample whose tiles end after u
  while (b < hi) {
    const int mid = (b + hi) >> 1;
    if (tend[mid] > u) hi = mid; else b = mid + 1;
  }
  const int t = u - (b > 0 ? tend[b - 1] : 0);
  const int q0 = a.q_off[b], q1 = a.q_off[b + 1], k0 = a.kv_off[b], k1 = a.kv_off[b + 1];
  const int nb = a.scratch_nch[b], rank = a.scratch_rank[b], max_items = a.max_items;
  const int tis = __builtin_ctz(a.tile_item), tls = __builtin_ctz(a.tile_loop);
  const bool qmode = a.mode == SCHED_QTILES;
  Item it;
  it.b = b; it.tile = t; it.aux = u;
  it.q0 = q0; it.lq = q1 - q0; it.kv0 = k0; it.lk = k1 - k0;
  it.lo = 0;
  it.hi = item_cost(a.mode, a.causal, a.win, it.lq, it.lk, t, tis, tls);
  it.slot = -1; it.chunk = 0;
  const int w = qmode ? nb - 1 - t : t;  // costliest tile first within the group
  Item* items = (Item*)a.items;
  const int32_t* gpre = a.scratch_gpre;
  for (int h0 = 0; h0 < H; h0 += 8) {
    int g0[8];  // the heads' group positions, loaded together before any item is stored
#pragma unroll
    for (int j = 0; j < 8; ++j) g0[j] = h0 + j < H ? gpre[rank * H + h0 + j] : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = h0 + j;
      if (h < H) {
        const int r = rank * H + h;
        const int pos = list_position(xtot, tgt, spre, dpre, group_xcd(r), g0[j] + w);
        it.h = h;
        if (pos >= 0 && pos < max_items) items[pos] = it;
      }
    }
  }
}

int persistent_grid(int cap, int per_cu) {
  static std::atomic<int> cus[64];  // compute units per device, looked up once
  int dev = 0, c = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) c = cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    if (dev >= 0 && dev < 64) cus[dev].store(c, std::memory_order_relaxed);
  }
  const int g = max(XCDS, (c * per_cu) / XCDS * XCDS);
  return cap < g ? cap : g;
}

bool sched_small(const SchedArgs& a) { return a.B <= SNT && (int64_t)a.B * a.H <= GCAP; }

// One workgroup per list (lists share the batch, so they all fit the LDS tables or none does).
// A list of at least DEFER_ITEMS possible items has its items written by sched_items_kernel
// (when no tile splits): one workgroup writing them all took 20-35 us on batches of a few
// hundred samples, mostly spent placing items one by one.
constexpr int64_t DEFER_ITEMS = 16384;

static hipError_t launch_lists(int n, const SchedArgs& a, const SchedArgs& b, const SchedArgs& c, hipStream_t s) {
  prof_before(PROF_SCHED, s);
  SchedLists lists;
  lists.l[0] = a;
  lists.l[1] = b;
  lists.l[2] = c;
  const bool small = sched_small(a);
  ItemsGrid grid;
  int wgs = 0;
  for (int i = 0; i < 3; ++i) {
    SchedArgs& l = lists.l[i];
    grid.first[i] = wgs;
    l.defer = i < n && small && l.H > 0 && (int64_t)l.max_items >= DEFER_ITEMS && l.scratch_at != nullptr;
    if (l.defer) wgs += (int)((l.max_items / l.H + ITEM_NT - 1) / ITEM_NT);  // max_items >= H * tiles
  }
  grid.first[3] = wgs;
  if (small)
    hipLaunchKernelGGL(sched_kernel<true>, dim3(n), dim3(SNT), 0, s, lists);
  else
    hipLaunchKernelGGL(sched_kernel<false>, dim3(n), dim3(SNT), 0, s, lists);
  if (wgs > 0) hipLaunchKernelGGL(sched_items_kernel, dim3(wgs), dim3(ITEM_NT), 0, s, lists, grid);
  prof_after(PROF_SCHED, s);
  return hipGetLastError();
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t s) { return launch_lists(1, a, a, a, s); }

hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t s) {
  return launch_lists(2, a, b, b, s);
}

hipError_t launch_sched3(const SchedArgs& a, const SchedArgs& b, const SchedArgs& c, hipStream_t s) {
  return launch_lists(3, a, b, c, s);
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
  constexpr int RBC = 1024;  // row blocks whose entry ranges one pass stages in LDS
  __shared__ int rlo[RBC], rhi[RBC];
  const int win = WIN ? a.win : 0;  // a compile-time zero without a window
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int c = blockIdx.y * 256 + threadIdx.x;
  const bool live = c < a.nb;  // threads past the table still join the barriers
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
    static_assert(BATCH == 16, "the load pins below name 16 registers");
    // Row block rb reaches diagonals up to 32 rb + 31 (clamped), so entry c sees only row blocks
    // rb >= (c - 31) / 32: the loop starts at the wave's first such block (its lowest c) and is
    // empty past the last row block. Blocks it skips would each have added +0.0.
    const int c_first = __builtin_amdgcn_readfirstlane(c);
    // With a sliding window a row block's first visited key tile starts at most KL - 1 keys
    // before its first query's window, so it wrote no diagonal above win + KL + 29: a wave whose
    // entries all lie above that sums nothing.
    const bool above_window = WIN && c_first > win + KL + 29;
    const int rb_begin = c_first > 32 * nrb - 1 || above_window ? nrb : max(0, (c_first - 31) / 32);
    if (a.split_slot == nullptr || hdr->n_split == 0) {
      // No split tiles: one row per row block. The clamped entry range each row block wrote is
      // staged in LDS by the workgroup (vector work, RBC row blocks per pass) rather than
      // recomputed per load by every wave in scalar code, which serialised on the scalar unit.
      // Each wave then issues a batch's loads (in bounds: the entry is clamped into the row,
      // no branches), and an entry outside its row block's range is cleared by a bit mask
      // (stale bits there may be anything, even NaN). The summation order is rb ascending.
      const int cl = min(c, nb - 1);
      const int wg_first = max(0, ((int)blockIdx.y * 256 - 31) / 32);
      for (int r0 = wg_first; r0 < nrb; r0 += RBC) {
        const int rn = min(RBC, nrb - r0);
        __syncthreads();  // the previous pass's range reads are done
        for (int i = threadIdx.x; i < rn; i += 256) {
          const int rb = r0 + i;
          int kf;
          const int nkt = qtile_cost<QI, KL>(rb / PER, Lq, Lk, a.causal, win, kf);
          int d_lo = 1, d_hi = 0;
          const bool any = chunk_range<KL>(rb, Lq, a.causal, win, kf, kf + nkt, d_lo, d_hi);
          rlo[i] = any ? clampi(d_lo, 0, nb - 1) : nb;
          rhi[i] = any ? clampi(d_hi, 0, nb - 1) : -1;
        }
        __syncthreads();
        for (int rb0 = max(r0, rb_begin); rb0 < r0 + rn; rb0 += BATCH) {
          int xi[BATCH];
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int rb = min(rb0 + u, r0 + rn - 1);
            const int64_t row = (int64_t)(tb + rb / PER) * PER + rb % PER;
            xi[u] = __float_as_int(a.part[((int64_t)h * a.part_rows + row) * nb + cl]);
          }
          // every load of the batch is issued before the first is used
          asm volatile("" ::"v"(xi[0]), "v"(xi[1]), "v"(xi[2]), "v"(xi[3]), "v"(xi[4]), "v"(xi[5]),
                       "v"(xi[6]), "v"(xi[7]));
          asm volatile("" ::"v"(xi[8]), "v"(xi[9]), "v"(xi[10]), "v"(xi[11]), "v"(xi[12]),
                       "v"(xi[13]), "v"(xi[14]), "v"(xi[15]));
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int i = min(rb0 + u, r0 + rn - 1) - r0;
            const bool keep = rb0 + u < r0 + rn && c >= rlo[i] && c <= rhi[i];
            acc += __int_as_float(xi[u] & (keep ? -1 : 0));
          }
        }
      }
    } else if (live) for (int rb0 = rb_begin; rb0 < nrb; rb0 += BATCH) {
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
        const float x = a.part[((int64_t)h * a.part_rows + row) * nb + c];
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
  if (live) a.part_bh[((int64_t)b * a.H + h) * a.nb + c] = acc;
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
