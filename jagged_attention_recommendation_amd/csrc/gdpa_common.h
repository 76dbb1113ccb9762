// Device-side building blocks shared by the gdpa kernels (gfx950 / CDNA4, wave64).
//
// Operand layouts of the matrix instructions used here (checked on the device with an in-bounds
// probe of the builtins):
//  * v_mfma_f32_32x32x16_bf16: lane l holds row (A) / column (B) l%32 and the 8 consecutive
//    k values 8*(l/32)..8*(l/32)+7. Accumulator register r of lane l is element
//    (row (r/4)*8 + 4*(l/32) + r%4, column l%32).
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands: bytes 0..15 of a lane belong to the
//    first 32-wide k block of the instruction and bytes 16..31 to the second; the e8m0 scale of
//    row m for k block kb is taken from lane m + 32*kb. Which k each byte is inside its block
//    does not matter as long as A and B agree.
//  * ds_read_b64_tr_b16: inside every group of 16 lanes, lane j receives element j%4 of the
//    8-byte chunks addressed by lanes j/4, j/4+4, j/4+8, j/4+12. Pointing lane 4t+q at
//    row (r0+t), column (c0+4q) of a row-major 16-bit tile therefore hands lane j the column
//    c0+j of rows r0..r0+3: a transposed read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define GDPA_LDS __attribute__((address_space(3)))

// Work item of the jagged scheduler: sample, tile index (of queries for forward / dQ, of keys
// for dK/dV), head, the canonical index of the (sample, tile), and the range [lo, hi) of
// inner-loop tiles the item covers (counted from the first tile the tile visits). A long tile
// split into n chunks has one item per chunk: slot is the chunk's partial-result slot (the
// tile's chunks use consecutive slots) and chunk packs the chunk index (low 16 bits) with n; an
// unsplit item has slot -1 and chunk 0. The sample's first query and key rows and its lengths
// ride along, so a workgroup learns everything about its item from one round trip instead of
// reading the offsets after the item.
struct Item {
  int b, tile, h, aux;
  int lo, hi, slot, chunk;
  int q0, lq, kv0, lk;
};

// Workspace header (first 256 bytes of every workspace).
struct WsHeader {
  int error;      // 0 ok, 1 bad q_offsets, 2 bad kv_offsets
  int n_items;    // items written by the scheduler
  int n_items2;   // second list (backward: key-tile items)
  int n_split;    // split tiles of the first list
  int n_split2;   // split tiles of the second list
  int chunk;      // inner tiles per chunk, first list (0: no splitting)
  int chunk2;     // inner tiles per chunk, second list
  int die_items[8];   // items placed on each die as their group's own (first list)
  int die_items2[8];  // same, second list
  int qctr[8];        // per-die claim counters of the persistent kernels (first list)
  int qctr2[8];       // same, second list
  int pad[25];
};
static_assert(sizeof(WsHeader) == 256, "header size");
static_assert(sizeof(Item) == 48, "item record size");

// The workgroup's item of list `which` (0: the header's n_items, 1: n_items2) and whether it
// exists. The header words and the item are loaded together and pinned before the test, so
// they cost one round trip (the compiler would otherwise load the error word, then the count,
// then the item, each after the previous test). The item slot is in bounds whatever the count;
// its contents are not used when the item does not exist.
__device__ __forceinline__ bool fetch_item(const void* hdr, const void* items, int which, Item& it) {
  const WsHeader* h = (const WsHeader*)hdr;
  it = ((const Item*)items)[blockIdx.x];
  const int err = h->error;
  const int n = which == 0 ? h->n_items : h->n_items2;
  asm volatile("" ::"s"(err), "s"(n), "s"(it.b), "s"(it.lk));
  return err == 0 && (int)blockIdx.x < n;
}

// Persistent consumption of an item list by a grid of a few workgroups per compute unit. The
// workgroups of die x (x = blockIdx.x % 8: the dispatcher places workgroup i on die i % 8) take
// that die's items, indices 8q + x for q < t_x, in increasing q, by counting on the die's claim
// counter in the header (cleared by the scheduler); as the list holds each die's items costliest
// first, this is the longest-first order of a dispatcher, without a workgroup launch per item.
// A workgroup claims its next item when it starts the current one and fetches that item's record
// during the current item, so moving on costs no memory round trip. When its die has no
// unclaimed item left, it takes items of the die with the most unclaimed ones (queue_steal).
struct ItemQueue {
  int* ctr0;         // the eight claim counters
  const int* items;  // the list, 12 words per item
  int n, die;        // list length; die whose items the workgroup claims
};

// Opens list `which` (0: first, 1: second) of the workspace; false if the scheduler failed.
__device__ __forceinline__ bool queue_open(const void* hdr, const void* items, int which, ItemQueue& q) {
  WsHeader* h = (WsHeader*)hdr;  // the claim counters are the only header words written here
  q.die = blockIdx.x & 7;
  q.ctr0 = which == 0 ? h->qctr : h->qctr2;
  q.items = (const int*)items;
  q.n = which == 0 ? h->n_items : h->n_items2;
  return h->error == 0;
}

// Claims the die's next item: its index for thread 0, -1 for the other threads.
__device__ __forceinline__ int queue_claim(const ItemQueue& q) {
  return threadIdx.x == 0 ? 8 * atomicAdd(q.ctr0 + q.die, 1) + q.die : -1;
}

// Items of die x in a list of n: t_x.
__device__ __forceinline__ int queue_die_items(int n, int x) { return (n >> 3) + (x < (n & 7) ? 1 : 0); }

// Called by the whole workgroup when its die has no unclaimed item: claims an item of the die
// with the most unclaimed items and moves the queue there. Returns the item's index, or n when
// no die has one left. The counters are read from the device-coherent level; a claim that loses
// a race (the die's last items went to others) looks again.
__device__ __forceinline__ int queue_steal(ItemQueue& q, GDPA_LDS int* slot) {
  for (;;) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int rem = 0;
      if (lane < 8) {
        const int c = __hip_atomic_load(q.ctr0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rem = queue_die_items(q.n, lane) - c;
      }
      int best = -1, best_rem = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int r = __builtin_amdgcn_readlane(rem, x);
        if (r > best_rem) {
          best_rem = r;
          best = x;
        }
      }
      int res = q.n;  // nothing left anywhere
      if (best >= 0) {
        res = -1 - best;  // lost the race on die best: look again
        if (lane == 0) {
          const int c = atomicAdd(q.ctr0 + best, 1);
          if (c < queue_die_items(q.n, best)) res = 8 * c + best;
        }
      }
      if (lane == 0) *slot = res;
    }
    __syncthreads();
    const int res = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();  // the slot may be written again
    if (res >= 0) {
      if (res < q.n) q.die = res & 7;
      return res;
    }
  }
}

// Lane l < 12 of the calling wave loads word l of item idx. It is always a load: an index past
// the list reads item 0 (a kernel runs only on a list with room for at least one), a record that
// is never used. A register that is only ever loaded into needs no wait before its next load;
// writing a constant into it instead made the compiler wait for every memory operation in
// flight, the next tile's loads included, at the first tile of every item.
__device__ __forceinline__ int queue_fetch(const ItemQueue& q, int idx) {
  const int lane = threadIdx.x & 63;
  const int i = idx < q.n ? idx : 0;
  return q.items[(int64_t)i * 12 + (lane < 12 ? lane : 11)];
}

// Starts bringing rows r0 .. r0 + 31 of head h of a jagged [rows, H, D] bf16 tensor (sample at
// row base, L rows) into the caches ahead of the item that will load them: direct loads of 16
// bytes per lane (whole rows, 64 / (D / 8) rows per instruction) into a 1 KiB LDS area that
// nothing reads. Rows at or past L lie outside the buffer resource and are not fetched.
template <int D>
__device__ __forceinline__ void prefetch_rows32(GDPA_LDS char* sink, const __bf16* src, int r0, int L,
                                                int base, int H, int h, int lane) {
  constexpr int RB = 2 * D;     // bytes per row
  constexpr int LPR = RB / 16;  // lanes per row
  constexpr int RPI = 64 / LPR; // rows per instruction
  const int n = min(32, L - r0);
  if (n <= 0) return;
  const __bf16* p = src + ((int64_t)(base + r0) * H + h) * D;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, ((n - 1) * H + 1) * RB, 0x00020000);
#pragma unroll
  for (int u = 0; u < 32 / RPI; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GDPA_LDS void*)sink, 16,
                                             (RPI * u + lane / LPR) * H * RB + (lane % LPR) * 16, 0, 0, 0);
}

// The record loaded by queue_fetch, as scalars.
__device__ __forceinline__ Item queue_record(int v) {
  Item it;
  it.b = __builtin_amdgcn_readlane(v, 0);
  it.tile = __builtin_amdgcn_readlane(v, 1);
  it.h = __builtin_amdgcn_readlane(v, 2);
  it.aux = __builtin_amdgcn_readlane(v, 3);
  it.lo = __builtin_amdgcn_readlane(v, 4);
  it.hi = __builtin_amdgcn_readlane(v, 5);
  it.slot = __builtin_amdgcn_readlane(v, 6);
  it.chunk = __builtin_amdgcn_readlane(v, 7);
  it.q0 = __builtin_amdgcn_readlane(v, 8);
  it.lq = __builtin_amdgcn_readlane(v, 9);
  it.kv0 = __builtin_amdgcn_readlane(v, 10);
  it.lk = __builtin_amdgcn_readlane(v, 11);
  return it;
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float GELU_C = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_A = 0.044715f;

enum { ACT_SOFTMAX = 0, ACT_GELU_TANH = 1, ACT_SILU = 2 };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Element-wise activations of GDPA in fp32, built on exp2 and the hardware reciprocal.
// GELU (tanh form): x/2 (1 + tanh(u)) with u = c (x + a x^3) equals x sigma(2u) =
// x / (1 + e^{-2u}), since 1 + tanh(u) = 2 sigma(2u); written that way it takes one exp2 and one
// reciprocal, and saturates without NaN (e^{-2u} = inf gives 0, e^{-2u} = 0 gives x).
// Its derivative is sigma + x sigma (1 - sigma) 2c (1 + 3 a x^2).
// SiLU: x sigma(x) = x / (1 + e^{-x}), derivative sigma (1 + x (1 - sigma)).
constexpr float GELU_K = -2.0f * GELU_C * LOG2E;       // -2u log2(e) = x (GELU_K + GELU_KA x^2)
constexpr float GELU_KA = GELU_K * GELU_A;
constexpr float GELU_D1 = 2.0f * GELU_C;                // 2c (1 + 3 a x^2) = GELU_D1 + GELU_D3 x^2
constexpr float GELU_D3 = 6.0f * GELU_C * GELU_A;

__device__ __forceinline__ float act_fwd(int act, float x) {
  if (act == ACT_GELU_TANH) {
    const float x2 = x * x;
    const float e = fast_exp2(x * fmaf(GELU_KA, x2, GELU_K));
    return x * fast_rcp(1.0f + e);
  }
  // silu
  const float e = fast_exp2(-LOG2E * x);
  return x * fast_rcp(1.0f + e);
}

// Value and derivative together (backward).
__device__ __forceinline__ void act_fwd_bwd(int act, float x, float& y, float& dy) {
  if (act == ACT_GELU_TANH) {
    const float x2 = x * x;
    const float e = fast_exp2(x * fmaf(GELU_KA, x2, GELU_K));
    const float sg = fast_rcp(1.0f + e);
    y = x * sg;
    dy = fmaf(y * (1.0f - sg), fmaf(GELU_D3, x2, GELU_D1), sg);
    return;
  }
  const float e = fast_exp2(-LOG2E * x);
  const float sg = fast_rcp(1.0f + e);
  y = x * sg;
  dy = sg * (1.0f + x * (1.0f - sg));
}

__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
  bf16x2 p0 = pack_bf16(v[0], v[1]), p1 = pack_bf16(v[2], v[3]);
  bf16x2 p2 = pack_bf16(v[4], v[5]), p3 = pack_bf16(v[6], v[7]);
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  i32x4 z = {0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

// Transposed read of 4 rows x 1 column (see the layout note above).
__device__ __forceinline__ i16x4 lds_read_tr(const GDPA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDPA_LDS i16x4*)p);
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Cross-half reductions of a wave64: v_permlane32_swap hands every lane l the pair
// {x[l % 32], x[l % 32 + 32]} (low half first), so combining the pair reduces over the two
// half-waves, with the same operand order in both halves (bitwise-identical results).
__device__ __forceinline__ float half_max(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane gets the same bits.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Sliding window of W keys (key j is valid for query i when j > i - W; W = 0: no window).
// First key tile (tiles of kl keys) that queries from q_lo on can reach.
__device__ __forceinline__ int win_first_ktile(int q_lo, int win, int kl) {
  return win > 0 ? max(0, q_lo - win + 1) / kl : 0;
}
// One past the last query tile (tiles of ql queries, nq of them) whose window reaches key k_hi.
__device__ __forceinline__ int win_end_qtile(int k_hi, int win, int ql, int nq) {
  return win > 0 ? min(nq, (k_hi + win - 1) / ql + 1) : nq;
}

}  // namespace gdpa
