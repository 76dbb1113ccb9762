// Host-side interface between the C-ABI entry points and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdpa {

struct Prob {
  int B, H, D, dtype, act, causal, nb;
  int win;  // sliding window W (0: none); only with causal, fp32 or bf16 D = 128
  int q_rows;  // shared query block: rows of Q / dQ (0: Q is jagged like O)
  int64_t total_q, total_kv;
  int max_q, max_kv;
  float scale;
};

enum { DT_F32 = 0, DT_BF16 = 1, DT_MX = 2 };

// Scheduler modes: items over query tiles (forward, dQ) or over key tiles (dK/dV).
enum { SCHED_QTILES = 0, SCHED_KTILES = 1 };

// Long tiles are split into chunks of inner tiles when splitting is on: the chunk length is
// T = max(SPLIT_MIN_TILES, ceil(total cost / nslot)), the mean load of nslot concurrent
// workgroups, and a tile of cost c > T becomes ceil(c / T) chunks. Split tiles each cost more
// than T, so there are at most total / T <= nslot of them and at most 2 * nslot chunks among
// them: the partial-result storage has a fixed size. A tile's cost is at most the total, so it
// has at most nslot chunks (Item::chunk keeps the count in 16 bits). nslot is SPLIT_NSLOT for
// the D = 128 kernels (two workgroups per compute unit) and twice that for D = 32 / 64, whose
// smaller tiles leave room for more workgroups per compute unit.
constexpr int SPLIT_NSLOT = 256;
constexpr int SPLIT_MIN_TILES = 8;

struct SchedArgs {
  const int32_t* q_off;
  const int32_t* kv_off;
  int B, H;
  int64_t total_q, total_kv;
  int mode, causal;
  int win;                   // sliding window W (0: none)
  int q_rows;                // shared query block: every Lq_b must be <= q_rows (0: no check)
  int tile_item, tile_loop;  // rows per item tile / rows per inner-loop tile
  int max_items;
  int list;                  // 0: first list of the header, 1: second list
  int split;                 // 1: split long tiles into chunks
  int nslot;                 // concurrent workgroups the chunk length aims at (see above)
  int defer;                 // set by the launch: a list without split tiles has its items
                             // written by a second, many-workgroup launch
  int32_t* tile_base;        // optional [B + 1]: canonical index of each sample's first tile
  int32_t* split_slot;       // optional [canonical tiles * H]: first slot of a split tile, or -1
  int32_t* split_cnt;        // [2 * nslot] chunk counters, indexed by a split tile's first slot
  void* ws_header;
  void* items;
  // per-sample and per-group values of batches larger than one scheduler workgroup holds in LDS
  // (sched_scratch_bytes); for a deferred list, what the item-writing launch reads: each sample's
  // item count, rank and inclusive tile end (scratch_at), and each group's first position
  unsigned long long* scratch_cost;  // [B]
  int32_t* scratch_nch;              // [B]
  int32_t* scratch_rank;             // [B]
  int32_t* scratch_at;               // [B]
  int32_t* scratch_gpre;             // [B * H]
};

// Workspace bytes of one list's scheduler scratch, and where its arrays sit in it.
inline size_t sched_scratch_bytes(int B, int H) {
  return (size_t)B * (8 + 3 * 4) + (size_t)B * H * 4;
}
inline void set_sched_scratch(SchedArgs& a, char* p, int B) {
  a.scratch_cost = (unsigned long long*)p;
  a.scratch_nch = (int32_t*)(p + (size_t)B * 8);
  a.scratch_rank = a.scratch_nch + B;
  a.scratch_at = a.scratch_rank + B;
  a.scratch_gpre = a.scratch_at + B;
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t s);
// Grid of a persistent kernel (ItemQueue) that holds per_cu workgroups per compute unit of the
// current device: at most cap workgroups (the list's capacity), a multiple of the 8 dies.
int persistent_grid(int cap, int per_cu);
hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t s);
// Three lists in one launch (a training forward's list and its backward's two).
hipError_t launch_sched3(const SchedArgs& a, const SchedArgs& b, const SchedArgs& c, hipStream_t s);

// Bias gradient reduction. The dQ kernels write, per (32-query row block, head), the diagonal
// sums of dS its queries produced (one row of NB floats, canonical row order); the reduction sums
// them per sample in row-block order (stage A, into part_bh [B, H, NB]) and then over samples in
// order (stage B).
// Rows of split dQ tiles go to the slot rows part_x[(slot * R + rb % R) * NB], one per chunk,
// and are summed in chunk order.
struct DbiasArgs {
  int part_rows;  // row blocks per head of part (head-major: [H, part_rows, NB])
  const int32_t* q_off;
  const int32_t* kv_off;
  const int32_t* tile_base;
  const int32_t* split_slot;  // [canonical tiles * H] or null
  const float* part;
  const float* part_x;
  float* part_bh;
  float* dbias;
  const void* hdr;
  int B, H, nb, causal;
  int win;        // sliding window W (0: none)
  int tile_rows;  // queries per dQ item
  int loop_rows;  // keys per dQ loop tile
};
hipError_t launch_dbias_reduce(const DbiasArgs& a, hipStream_t s);

// Upper bound on the number of items the scheduler can emit (slots: chunk slots of the list when
// it splits, else 0).
inline int64_t items_bound(int64_t total_rows, int B, int H, int tile, int slots) {
  return (int64_t)H * ((total_rows + tile - 1) / tile + (int64_t)B) + slots;
}

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const uint8_t* qs;
  const uint8_t* ks;
  const uint8_t* vs;
  const int32_t* q_off;
  const int32_t* kv_off;
  const float* bias;
  void* O;
  float* lse;
  const void* hdr;
  const void* items;
  int32_t* split_cnt;  // chunk counters of split tiles
  float* part_o;   // split chunks: [2 * nslot][BM][D] fp32 unnormalised output
  float* part_ml;  // split chunks (softmax): [2 * nslot][2][BM] running max (log2 units), sum
  int H, nb;
  int win;         // sliding window W (0: none)
  int q_shared;    // 1: Q is one block read by every sample (local query i reads row i)
  float scale;
};

// Rows of queries per forward work item, per element type.
constexpr int FWD_BM_BF16 = 128;
constexpr int FWD_BN_BF16 = 64;
constexpr int F32_BM = 64;
constexpr int F32_BN = 64;

// Largest bias window (floats) a kernel stages in LDS; wider windows are read from global memory.
constexpr int BIAS_WMAX = 4096;

hipError_t launch_fwd_bf16(const Prob& p, const FwdArgs& a, int grid, hipStream_t s);
hipError_t launch_fwd_mx(const Prob& p, const FwdArgs& a, int grid, hipStream_t s);
// Exact MX-fp8 -> bf16 dequantisation of a [rows, H, D] tensor (D = 128).
hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, void* out, int64_t rows,
                             int H, int D, hipStream_t s);
hipError_t launch_fwd_f32(const Prob& p, const FwdArgs& a, int grid, hipStream_t s);

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;
  const int32_t* q_off;
  const int32_t* kv_off;
  const float* bias;
  void* dQ;
  void* dK;
  void* dV;
  float* dbias;
  float* Dvec;           // [total_q, H] softmax row term
  const void* hdr;
  const void* items_q;   // query-tile items (dQ)
  const void* items_k;   // key-tile items (dK/dV)
  float* dbias_part;     // [H, part_rows, NB] per 32-query row block diagonal sums of dS
  int part_rows;         // row blocks the partial-row buffer holds per head
  float* dbias_part_x;   // split chunks: [2 * nslot * QI / 32, NB]
  int32_t* split_cnt_q;  // chunk counters of split query tiles
  int32_t* split_cnt_k;  // chunk counters of split key tiles
  const int32_t* tile_base;  // [B + 1] canonical index of each sample's first query tile
  float* part_dq;        // split chunks: [2 * nslot][QI][D] fp32
  float* part_dk;        // split chunks: [2 * nslot][KI][D] fp32
  float* part_dv;
  int H, nb;
  int win;               // sliding window W (0: none)
  int q_shared;          // 1: Q is one block read by every sample (local query i reads row i)
  float* dq_f32;         // shared Q: per-sample dQ, fp32 scaled, at O's rows ([total_q, H, D]);
                         // null: dQ is written in place in bf16
  float scale;
};

// Shared query block: dQ[i, h] = sum over samples b with Lq_b > i of dq_f32[q_off[b] + i, h],
// summed in a fixed order, rounded once to bf16 (or kept in fp32 for fp32 problems).
struct DqSharedArgs {
  const int32_t* q_off;
  const float* part;
  void* dQ;
  const void* hdr;
  int B, H, D, q_rows;
  int f32_out;  // 1: dQ is fp32, else bf16
};
hipError_t launch_dq_shared_reduce(const DqSharedArgs& a, hipStream_t s);

constexpr int BWD_Q_ITEM = 128;  // queries per dQ work item (bf16)
constexpr int BWD_K_LOOP = 64;   // keys per tile in the dQ loop (bf16)
constexpr int BWD_K_ITEM = 128;  // keys per dK/dV work item (bf16)
constexpr int BWD_Q_LOOP = 64;   // queries per tile in the dK/dV loop (bf16)

// The scheduler divides by tile sizes with shifts: every tile size is a power of two.
constexpr bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
static_assert(pow2(FWD_BM_BF16) && pow2(FWD_BN_BF16) && pow2(F32_BM) && pow2(F32_BN) &&
                  pow2(BWD_Q_ITEM) && pow2(BWD_K_LOOP) && pow2(BWD_K_ITEM) && pow2(BWD_Q_LOOP),
              "tile sizes must be powers of two");

hipError_t launch_bwd_bf16(const Prob& p, const BwdArgs& a, int grid_q, int grid_k, hipStream_t s);

// Which lists of this problem take split items (the last chunk of a split tile combines the
// tile, see gdpa_split.h): forward and dQ on every bf16 kernel (the D = 32 / 64 dQ kernel only
// without a bias table), dK/dV on the D = 128 kernel.
inline bool split_fwd(const Prob& p) { return p.dtype == DT_BF16; }
inline bool split_dq(const Prob& p) { return p.dtype == DT_BF16 && (p.D == 128 || p.nb == 0); }
inline bool split_dkdv(const Prob& p) { return p.dtype == DT_BF16 && p.D == 128; }
inline int split_nslot(const Prob& p) { return p.D == 128 ? SPLIT_NSLOT : 2 * SPLIT_NSLOT; }
inline int split_slots(const Prob& p) { return 2 * split_nslot(p); }
hipError_t launch_bwd_f32(const Prob& p, const BwdArgs& a, int grid_q, int grid_k, hipStream_t s);

// Block-aligned attention: fixed blocks of BLOCK_TOKENS consecutive tokens per sample, each
// attending only within itself, with rotary embeddings of Q and K (gdpa_block.hip). Items are the
// scheduler's query tiles of BLOCK_TOKENS rows.
constexpr int BLOCK_TOKENS = 64;
static_assert(pow2(BLOCK_TOKENS), "tile sizes must be powers of two");
struct BlockArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const int32_t* off;  // [B + 1] sample offsets (Q, K, V, O share them)
  void* O;
  void* dQ;
  void* dK;
  void* dV;
  const void* hdr;
  const void* items;
  int H;
  float scale;
  double rope_log2_base;  // log2 of the rotary base (pair m turns by p * base^(-2m/D))
};
hipError_t launch_block(int act, bool causal, bool rope, const BlockArgs& a, int grid, bool bwd,
                        hipStream_t s);

// Profiling hook: brackets launches of one kernel with HIP events (see gdpa_profile_start).
enum { PROF_FWD = 0, PROF_DQ = 1, PROF_DKDV = 2, PROF_SCHED = 3, PROF_BLOCK_FWD = 4,
       PROF_BLOCK_BWD = 5 };
void prof_before(int kernel, hipStream_t s);
void prof_after(int kernel, hipStream_t s);

}  // namespace gdpa
