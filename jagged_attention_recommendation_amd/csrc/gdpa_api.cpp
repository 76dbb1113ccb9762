// C-ABI entry points of libgdpa.so (declared in include/gdpa.h): argument validation, workspace
// carving and kernel launches on the caller's stream. No device memory is allocated here and no
// call synchronises the host, except gdpa_read_device_error().
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "gdpa.h"
#include "gdpa_common.h"
#include "gdpa_internal.h"

using namespace gdpa;

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// The window the kernels see. A window of W keys drops key j for query i only when j <= i - W,
// which needs i >= W; when W is at least every sample's query count (Lq <= total_q, and
// Lq <= max_q when that bound is given) it drops nothing and is treated as no window. The kernels
// then only form positions plus W with W < total_q, which stays inside int32 because
// check_problem() bounds total_q + total_kv.
int32_t effective_window(const gdpa_problem* p) {
  if (p->window <= 0) return 0;
  if ((int64_t)p->window >= p->total_q) return 0;
  if (p->max_q > 0 && p->window >= p->max_q) return 0;
  return p->window;
}

int32_t check_problem(const gdpa_problem* p) {
  if (p == nullptr) return GDPA_EINVAL;
  if (p->B < 0 || p->H < 1 || p->total_q < 0 || p->total_kv < 0) return GDPA_EINVAL;
  if (p->total_q >= (int64_t)1 << 31 || p->total_kv >= (int64_t)1 << 31) return GDPA_EINVAL;
  if (p->dtype < GDPA_F32 || p->dtype > GDPA_MXFP8_E4M3) return GDPA_EINVAL;
  if (p->act < GDPA_ACT_SOFTMAX || p->act > GDPA_ACT_SILU) return GDPA_EINVAL;
  if (p->causal != 0 && p->causal != 1) return GDPA_EINVAL;
  if (p->bias_buckets < 0 || p->max_q < 0 || p->max_kv < 0) return GDPA_EINVAL;
  if (!isfinite(p->scale)) return GDPA_EINVAL;
  // the bf16 and MX kernels take row maxima on unscaled scores, which needs scale > 0
  if (p->dtype != GDPA_F32 && !(p->scale > 0.0f)) return GDPA_ENOTSUP;
  if (p->D != 32 && p->D != 64 && p->D != 128) return GDPA_ENOTSUP;
  if (p->dtype == GDPA_MXFP8_E4M3 && p->D != 128) return GDPA_ENOTSUP;
  if (p->window < 0) return GDPA_EINVAL;
  // sliding windows: causal attention on the fp32 and bf16 kernels
  if (p->window > 0 && (p->causal != 1 || p->dtype == GDPA_MXFP8_E4M3)) return GDPA_ENOTSUP;
  // window arithmetic adds a key or query position to W in int32
  if (effective_window(p) > 0 && p->total_q + p->total_kv > INT32_MAX - 1024) return GDPA_ENOTSUP;
  // a shared query block: bf16 kernels, max_q rows
  if (p->q_shared != 0 && p->q_shared != 1) return GDPA_EINVAL;
  if (p->q_shared && p->max_q < 1) return GDPA_EINVAL;
  if (p->q_shared && p->dtype == GDPA_MXFP8_E4M3) return GDPA_ENOTSUP;
  // element counts must fit the kernels' 64-bit addressing and the scheduler's int32 counters
  if ((int64_t)p->H * p->D > (1 << 20)) return GDPA_ENOTSUP;
  return GDPA_OK;
}

Prob to_prob(const gdpa_problem* p) {
  Prob r;
  r.B = p->B; r.H = p->H; r.D = p->D; r.dtype = p->dtype; r.act = p->act; r.causal = p->causal;
  r.nb = p->bias_buckets; r.total_q = p->total_q; r.total_kv = p->total_kv;
  r.max_q = p->max_q; r.max_kv = p->max_kv; r.scale = p->scale; r.win = effective_window(p);
  r.q_rows = p->q_shared ? p->max_q : 0;
  return r;
}

int fwd_tile_rows(int dtype) { return dtype == GDPA_F32 ? F32_BM : FWD_BM_BF16; }
int fwd_loop_rows(int dtype) { return dtype == GDPA_F32 ? F32_BN : FWD_BN_BF16; }
int bwd_q_item(int dtype) { return dtype == GDPA_F32 ? F32_BM : BWD_Q_ITEM; }
int bwd_k_loop(int dtype) { return dtype == GDPA_F32 ? F32_BN : BWD_K_LOOP; }
int bwd_k_item(int dtype) { return dtype == GDPA_F32 ? F32_BN : BWD_K_ITEM; }
int bwd_q_loop(int dtype) { return dtype == GDPA_F32 ? F32_BM : BWD_Q_LOOP; }

struct FwdLayout {
  size_t header, items, sched, split_cnt, part_o, part_ml, total;
  int64_t max_items;
  bool split;
  int slots;  // chunk slots (0 without splitting)
};

FwdLayout fwd_layout(const gdpa_problem* p) {
  FwdLayout L;
  const Prob pr = to_prob(p);
  L.split = split_fwd(pr);
  L.slots = L.split ? split_slots(pr) : 0;
  L.max_items = items_bound(p->total_q, p->B, p->H, fwd_tile_rows(p->dtype), L.slots);
  L.header = 0;
  L.items = ALIGN;
  L.sched = L.items + align_up((size_t)L.max_items * sizeof(Item));
  L.split_cnt = L.sched + align_up(sched_scratch_bytes(p->B, p->H));
  L.part_o = L.part_ml = L.total = L.split_cnt;
  if (L.split) {
    const size_t rows = (size_t)L.slots * fwd_tile_rows(p->dtype);
    L.part_o = L.split_cnt + align_up((size_t)L.slots * sizeof(int32_t));
    L.part_ml = L.part_o + align_up(rows * p->D * sizeof(float));
    L.total = L.part_ml + align_up(rows * 2 * sizeof(float));
  }
  return L;
}

struct BwdLayout {
  size_t header, items_q, items_k, sched_q, sched_k, dvec, tile_base, part, part_bh, split_cnt_q, split_cnt_k,
      split_slot, part_dq, part_dk, part_dv, part_x, dq_f32, total;
  int64_t max_q_items, max_k_items, max_qtiles;
  bool split, split_q, split_k;  // split storage present / per list
  int slots;                     // chunk slots of each list (0 without splitting)
};

BwdLayout bwd_layout(const gdpa_problem* p) {
  BwdLayout L;
  const Prob pr = to_prob(p);
  L.split_q = split_dq(pr);
  L.split_k = split_dkdv(pr);
  L.split = L.split_q || L.split_k;
  L.slots = L.split ? split_slots(pr) : 0;
  const int tq = bwd_q_item(p->dtype), tk = bwd_k_item(p->dtype);
  L.max_q_items = items_bound(p->total_q, p->B, p->H, tq, L.split_q ? L.slots : 0);
  L.max_k_items = items_bound(p->total_kv, p->B, p->H, tk, L.split_k ? L.slots : 0);
  L.max_qtiles = (p->total_q + tq - 1) / tq + p->B;
  L.header = 0;
  L.items_q = ALIGN;
  L.items_k = L.items_q + align_up((size_t)L.max_q_items * sizeof(Item));
  L.sched_q = L.items_k + align_up((size_t)L.max_k_items * sizeof(Item));
  L.sched_k = L.sched_q + align_up(sched_scratch_bytes(p->B, p->H));
  L.dvec = L.sched_k + align_up(sched_scratch_bytes(p->B, p->H));
  L.tile_base = L.dvec + align_up((size_t)p->total_q * p->H * sizeof(float));
  L.part = L.tile_base + align_up((size_t)(p->B + 1) * sizeof(int32_t));
  L.part_bh = L.part;
  size_t end = L.part;
  if (p->bias_buckets > 0) {
    // one partial row per 32-query row block and head, then one per sample and head
    const size_t rows = (size_t)L.max_qtiles * (tq / 32);
    L.part_bh = L.part + align_up(rows * p->H * p->bias_buckets * sizeof(float));
    end = L.part_bh + align_up((size_t)p->B * p->H * p->bias_buckets * sizeof(float));
  }
  L.split_cnt_q = L.split_cnt_k = L.split_slot = L.part_dq = L.part_dk = L.part_dv = L.part_x = end;
  if (L.split) {
    // chunk counters of both lists, the per-(tile, head) slot table, the chunks' partial rows
    L.split_cnt_q = end;
    L.split_cnt_k = L.split_cnt_q + align_up((size_t)L.slots * sizeof(int32_t));
    L.split_slot = L.split_cnt_k + align_up((size_t)L.slots * sizeof(int32_t));
    L.part_dq = L.split_slot + align_up((size_t)L.max_qtiles * p->H * sizeof(int32_t));
    // partial rows only for the lists that split
    const size_t nq = L.split_q ? L.slots : 0, nk = L.split_k ? L.slots : 0;
    L.part_dk = L.part_dq + align_up(nq * tq * p->D * sizeof(float));
    L.part_dv = L.part_dk + align_up(nk * tk * p->D * sizeof(float));
    L.part_x = L.part_dv + align_up(nk * tk * p->D * sizeof(float));
    end = L.part_x;
    if (p->bias_buckets > 0) end += align_up(nq * (tq / 32) * p->bias_buckets * sizeof(float));
  }
  // shared query block: every sample's dQ in fp32 at O's rows, summed over samples afterwards
  L.dq_f32 = end;
  if (p->q_shared) end += align_up((size_t)p->total_q * p->H * p->D * sizeof(float));
  L.total = end;
  return L;
}

// Host-checkable arguments of a backward call (Q, K, V are the bf16 / fp32 tensors the kernels
// read; for the MX backward they are the dequantised copies, checked with placeholders).
int32_t check_bwd_args(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                       const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                       const int32_t* kv_offsets, const float* bias, const void* dQ,
                       const void* dK, const void* dV, const float* dbias, const void* workspace) {
  if (!q_offsets || !kv_offsets || !workspace) return GDPA_EINVAL;
  if (p->total_q > 0 && (!Q || !dO || !dQ)) return GDPA_EINVAL;
  if (p->q_shared && (!Q || !dQ)) return GDPA_EINVAL;  // dQ is written even with no queries
  if (p->total_kv > 0 && (!K || !V || !dK || !dV)) return GDPA_EINVAL;
  const bool softmax = p->act == GDPA_ACT_SOFTMAX;
  if (softmax && p->total_q > 0 && (!O || !lse)) return GDPA_EINVAL;
  if ((p->bias_buckets > 0) != (bias != nullptr)) return GDPA_EINVAL;
  if ((p->bias_buckets > 0) != (dbias != nullptr)) return GDPA_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(workspace))
    return GDPA_EINVAL;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)bias & 3u) || ((uintptr_t)dbias & 3u) ||
      ((uintptr_t)q_offsets & 3u) || ((uintptr_t)kv_offsets & 3u))
    return GDPA_EINVAL;
  return GDPA_OK;
}

// MX backward: Q, K, V dequantised exactly to bf16 at the start of the workspace, then the bf16
// backward's own workspace.
struct MxBwdLayout {
  size_t q, k, v, bwd, total;
};

gdpa_problem bf16_view(const gdpa_problem* p) {
  gdpa_problem r = *p;
  r.dtype = GDPA_BF16;
  return r;
}

MxBwdLayout mx_bwd_layout(const gdpa_problem* p) {
  MxBwdLayout L;
  const size_t row = (size_t)p->H * p->D * 2;
  L.q = 0;
  L.k = L.q + align_up((size_t)p->total_q * row);
  L.v = L.k + align_up((size_t)p->total_kv * row);
  L.bwd = L.v + align_up((size_t)p->total_kv * row);
  const gdpa_problem pb = bf16_view(p);
  L.total = L.bwd + bwd_layout(&pb).total;
  return L;
}

// ---- scratch of gdpa_fwd_static: one fixed buffer per GPU in place of a caller workspace.
// Host code never uses the array's name as an address (on the host it only names the symbol):
// every launch takes the device address that hipGetSymbolAddress returned for the current GPU.
static __device__ __align__(256) char scratch[GDPA_STATIC_SCRATCH_BYTES];

constexpr int SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_DEVICES];  // device address of `scratch` per GPU, null until looked up

// Device address of `scratch` on the current GPU: looked up once per GPU, with that GPU current.
int32_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDPA_EHIP;
  if (dev < 0 || dev >= SCRATCH_DEVICES) return GDPA_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return GDPA_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDPA_OK;
}

// ---- profiling hook state
constexpr int PROF_KERNELS = 6;
constexpr int PROF_MAX = 1024;
// Launches may come from several host threads: the mask and the per-kernel slot counters are
// atomic, and the slot a launch claimed in prof_before is handed to prof_after (same thread,
// same launch) through a thread-local.
struct ProfState {
  std::atomic<int> mask{0};
  std::atomic<int> n[PROF_KERNELS];
  bool created = false;
  hipEvent_t ev[PROF_KERNELS][2 * PROF_MAX];
};
ProfState g_prof;
thread_local int t_prof_slot[PROF_KERNELS] = {-1, -1, -1, -1, -1, -1};
static_assert(PROF_KERNELS == 6, "t_prof_slot initialiser");

// A second stream (default priority, non-blocking) and two events per device and host thread,
// created on first use and kept until the thread ends: the backward runs the bias-gradient
// reduction on it beside the dK/dV kernel (fork after dQ, join before returning). Per thread, so
// that concurrent callers never share an event between its record and its wait. Null if any of
// them cannot be created; the caller then stays on its own stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};
thread_local SideStream t_side[64];

SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = t_side[dev];
  if (!ss.tried) {
    ss.tried = true;
    // fork / join order work between two streams of one device: a device-scope release is enough
    const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, ef) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, ef) != hipSuccess)
      ss.s = nullptr;
  }
  return ss.s != nullptr ? &ss : nullptr;
}

int32_t map_hip(hipError_t e) {
  if (e == hipSuccess) return GDPA_OK;
  if (e == hipErrorNotSupported) return GDPA_ENOTSUP;
  return GDPA_EHIP;
}

}  // namespace

namespace gdpa {
void prof_before(int kernel, hipStream_t s) {
  t_prof_slot[kernel] = -1;
  if (!(g_prof.mask.load(std::memory_order_acquire) >> kernel & 1)) return;
  const int i = g_prof.n[kernel].fetch_add(1, std::memory_order_relaxed);
  if (i >= PROF_MAX) return;
  t_prof_slot[kernel] = i;
  (void)hipEventRecord(g_prof.ev[kernel][2 * i], s);
}
void prof_after(int kernel, hipStream_t s) {
  const int i = t_prof_slot[kernel];
  if (i < 0) return;
  (void)hipEventRecord(g_prof.ev[kernel][2 * i + 1], s);
  t_prof_slot[kernel] = -1;
}
}  // namespace gdpa

extern "C" {

int32_t gdpa_profile_start(int32_t mask) {
  if (mask < 0 || mask >= (1 << PROF_KERNELS)) return GDPA_EINVAL;
  if (!g_prof.created) {
    for (int k = 0; k < PROF_KERNELS; ++k)
      for (int i = 0; i < 2 * PROF_MAX; ++i)
        // timing only: no system-scope fence (no cache writeback and invalidation around the
        // timed kernels, which would slow them and the work after them)
        if (hipEventCreateWithFlags(&g_prof.ev[k][i], hipEventDisableSystemFence) != hipSuccess)
          return GDPA_EHIP;
    g_prof.created = true;
  }
  for (int k = 0; k < PROF_KERNELS; ++k) g_prof.n[k].store(0, std::memory_order_relaxed);
  g_prof.mask.store(mask, std::memory_order_release);
  return GDPA_OK;
}

int32_t gdpa_profile_read(int32_t kernel, int32_t* launches, double* total_ms) {
  if (!launches || !total_ms || kernel < 0 || kernel >= PROF_KERNELS) return GDPA_EINVAL;
  double tot = 0.0;
  const int n = std::min(g_prof.n[kernel].load(std::memory_order_acquire), PROF_MAX);
  for (int i = 0; i < n; ++i) {
    float ms = 0.0f;
    if (hipEventSynchronize(g_prof.ev[kernel][2 * i + 1]) != hipSuccess) return GDPA_EHIP;
    if (hipEventElapsedTime(&ms, g_prof.ev[kernel][2 * i], g_prof.ev[kernel][2 * i + 1]) !=
        hipSuccess)
      return GDPA_EHIP;
    tot += ms;
  }
  *launches = n;
  *total_ms = tot;
  return GDPA_OK;
}

int32_t gdpa_profile_stop(void) {
  g_prof.mask.store(0, std::memory_order_release);
  return GDPA_OK;
}

int32_t gdpa_abi_version(void) { return GDPA_ABI_VERSION; }

const char* gdpa_status_string(int32_t s) {
  switch (s) {
    case GDPA_OK: return "ok";
    case GDPA_EINVAL: return "invalid argument";
    case GDPA_ENOTSUP: return "unsupported configuration";
    case GDPA_EWORKSPACE: return "workspace too small";
    case GDPA_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t gdpa_workspace_size(const gdpa_problem* p, int32_t for_bwd, size_t* bytes) {
  if (bytes == nullptr) return GDPA_EINVAL;
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (for_bwd && p->dtype == GDPA_MXFP8_E4M3) *bytes = mx_bwd_layout(p).total;
  else *bytes = for_bwd ? bwd_layout(p).total : fwd_layout(p).total;
  return GDPA_OK;
}

// ---- plans. gdpa_fwd_plan_bwd records, per backward workspace and device, the problem and the
// offset pointers it scheduled; gdpa_bwd_planned runs only on a workspace whose record matches
// its own arguments, and uses the record up; gdpa_bwd (which rebuilds the lists) forgets it.
struct PlanRec {
  const void* ws;
  int dev;
  gdpa_problem p;
  const int32_t* q_off;
  const int32_t* kv_off;
};
std::mutex g_plan_mu;
std::vector<PlanRec> g_plans;

bool same_problem(const gdpa_problem& a, const gdpa_problem& b) {
  return a.B == b.B && a.H == b.H && a.D == b.D && a.dtype == b.dtype && a.total_q == b.total_q &&
         a.total_kv == b.total_kv && a.max_q == b.max_q && a.max_kv == b.max_kv && a.act == b.act &&
         a.causal == b.causal && a.scale == b.scale && a.bias_buckets == b.bias_buckets &&
         a.window == b.window && a.q_shared == b.q_shared;
}

int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

void plan_record(const void* ws, const gdpa_problem* p, const int32_t* q_off, const int32_t* kv_off) {
  const PlanRec rec{ws, current_device(), *p, q_off, kv_off};
  std::lock_guard<std::mutex> lock(g_plan_mu);
  for (PlanRec& r : g_plans)
    if (r.ws == ws && r.dev == rec.dev) {
      r = rec;
      return;
    }
  if (g_plans.size() >= 4096) g_plans.erase(g_plans.begin());  // bounded: the oldest goes
  g_plans.push_back(rec);
}

// Removes the record of ws on this device; true if it matched the given problem and offsets.
bool plan_take(const void* ws, const gdpa_problem* p, const int32_t* q_off, const int32_t* kv_off) {
  const int dev = current_device();
  std::lock_guard<std::mutex> lock(g_plan_mu);
  for (size_t i = 0; i < g_plans.size(); ++i) {
    const PlanRec& r = g_plans[i];
    if (r.ws != ws || r.dev != dev) continue;
    const bool ok = same_problem(r.p, *p) && r.q_off == q_off && r.kv_off == kv_off;
    g_plans.erase(g_plans.begin() + i);
    return ok;
  }
  return false;
}

// The backward's two scheduler lists in workspace ws (layout L): query-tile items (dQ, D, bias
// partials) and key-tile items (dK, dV).
static void bwd_sched_args(const gdpa_problem* p, const Prob& pr, const BwdLayout& L, char* ws,
                           const int32_t* q_offsets, const int32_t* kv_offsets, SchedArgs& sq,
                           SchedArgs& sk) {
  const int tq = bwd_q_item(p->dtype), tk = bwd_k_item(p->dtype);
  SchedArgs sa;
  sa.q_off = q_offsets; sa.kv_off = kv_offsets; sa.B = p->B; sa.H = p->H;
  sa.total_q = p->total_q; sa.total_kv = p->total_kv; sa.causal = p->causal;
  sa.win = pr.win; sa.q_rows = pr.q_rows; sa.ws_header = ws + L.header;
  sa.nslot = split_nslot(pr);
  sq = sa;
  sk = sa;
  sq.split = L.split_q ? 1 : 0;
  sk.split = L.split_k ? 1 : 0;
  sq.mode = SCHED_QTILES; sq.tile_item = tq; sq.tile_loop = bwd_k_loop(p->dtype);
  sq.max_items = (int)L.max_q_items; sq.list = 0;
  sq.tile_base = (int32_t*)(ws + L.tile_base); sq.items = ws + L.items_q;
  sq.split_cnt = (int32_t*)(ws + L.split_cnt_q);
  sq.split_slot = L.split_q && p->bias_buckets > 0 ? (int32_t*)(ws + L.split_slot) : nullptr;
  sk.mode = SCHED_KTILES; sk.tile_item = tk; sk.tile_loop = bwd_q_loop(p->dtype);
  sk.max_items = (int)L.max_k_items; sk.list = 1;
  sk.tile_base = nullptr; sk.items = ws + L.items_k;
  sk.split_cnt = (int32_t*)(ws + L.split_cnt_k);
  sk.split_slot = nullptr;
  set_sched_scratch(sq, ws + L.sched_q, p->B);
  set_sched_scratch(sk, ws + L.sched_k, p->B);
}

// gdpa_fwd, and with bwd_ws also the backward's item lists (gdpa_fwd_plan_bwd).
static int32_t fwd_impl(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                        const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias, void* O,
                        float* lse, void* workspace, size_t workspace_bytes, void* bwd_ws,
                        size_t bwd_ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (!q_offsets || !kv_offsets || !workspace) return GDPA_EINVAL;
  if (p->total_q > 0 && (!Q || !O)) return GDPA_EINVAL;
  if (p->total_kv > 0 && (!K || !V)) return GDPA_EINVAL;
  if ((p->bias_buckets > 0) != (bias != nullptr)) return GDPA_EINVAL;
  const bool mx = p->dtype == GDPA_MXFP8_E4M3;
  if (mx && ((p->total_q > 0 && !q_scale) || (p->total_kv > 0 && (!k_scale || !v_scale))))
    return GDPA_EINVAL;
  if (!mx && (q_scale || k_scale || v_scale)) return GDPA_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
    return GDPA_EINVAL;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)bias & 3u) || ((uintptr_t)q_offsets & 3u) ||
      ((uintptr_t)kv_offsets & 3u))
    return GDPA_EINVAL;
  const Prob pr = to_prob(p);
  const FwdLayout L = fwd_layout(p);
  if (workspace_bytes < L.total) return GDPA_EWORKSPACE;
  if (L.max_items > INT32_MAX) return GDPA_ENOTSUP;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  SchedArgs sa;
  sa.q_off = q_offsets; sa.kv_off = kv_offsets; sa.B = p->B; sa.H = p->H;
  sa.total_q = p->total_q; sa.total_kv = p->total_kv; sa.mode = SCHED_QTILES;
  sa.causal = p->causal; sa.win = pr.win; sa.q_rows = pr.q_rows;
  sa.tile_item = fwd_tile_rows(p->dtype);
  sa.tile_loop = fwd_loop_rows(p->dtype); sa.max_items = (int)L.max_items; sa.list = 0;
  sa.split = L.split ? 1 : 0; sa.nslot = split_nslot(pr);
  sa.tile_base = nullptr; sa.split_slot = nullptr;
  sa.ws_header = ws + L.header; sa.items = ws + L.items;
  sa.split_cnt = (int32_t*)(ws + L.split_cnt);
  set_sched_scratch(sa, ws + L.sched, p->B);
  hipError_t e;
  if (bwd_ws != nullptr) {
    // the backward's lists in workgroups of their own, beside the forward's
    if (!aligned16(bwd_ws)) return GDPA_EINVAL;
    const BwdLayout LB = bwd_layout(p);
    if (bwd_ws_bytes < LB.total) return GDPA_EWORKSPACE;
    const uintptr_t f0 = (uintptr_t)workspace, b0 = (uintptr_t)bwd_ws;
    if (f0 < b0 + LB.total && b0 < f0 + L.total) return GDPA_EINVAL;  // the two must not overlap
    if (LB.max_q_items > INT32_MAX || LB.max_k_items > INT32_MAX) return GDPA_ENOTSUP;
    SchedArgs sq, sk;
    bwd_sched_args(p, pr, LB, (char*)bwd_ws, q_offsets, kv_offsets, sq, sk);
    e = launch_sched3(sa, sq, sk, s);
    if (e == hipSuccess) plan_record(bwd_ws, p, q_offsets, kv_offsets);
  } else {
    e = launch_sched(sa, s);
  }
  if (e != hipSuccess) return map_hip(e);

  FwdArgs fa;
  fa.Q = Q; fa.K = K; fa.V = V; fa.qs = q_scale; fa.ks = k_scale; fa.vs = v_scale;
  fa.q_off = q_offsets; fa.kv_off = kv_offsets; fa.bias = bias; fa.O = O;
  fa.lse = p->act == GDPA_ACT_SOFTMAX ? lse : nullptr;
  fa.hdr = ws + L.header; fa.items = ws + L.items; fa.H = p->H; fa.nb = p->bias_buckets;
  fa.scale = p->scale; fa.win = pr.win; fa.q_shared = p->q_shared; fa.split_cnt = (int32_t*)(ws + L.split_cnt);
  fa.part_o = (float*)(ws + L.part_o); fa.part_ml = (float*)(ws + L.part_ml);
  const int grid = (int)L.max_items;
  if (p->dtype == GDPA_F32) e = launch_fwd_f32(pr, fa, grid, s);
  else if (p->dtype == GDPA_BF16) e = launch_fwd_bf16(pr, fa, grid, s);
  else e = launch_fwd_mx(pr, fa, grid, s);
  return map_hip(e);
}

int32_t gdpa_fwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                 const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                 const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias, void* O,
                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(p, Q, K, V, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, O, lse,
                  workspace, workspace_bytes, nullptr, 0, stream);
}

int32_t gdpa_fwd_plan_bwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                          void* O, float* lse, void* workspace, size_t workspace_bytes,
                          void* bwd_workspace, size_t bwd_workspace_bytes, void* stream) {
  const int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (p->dtype == GDPA_MXFP8_E4M3) return GDPA_ENOTSUP;
  if (!bwd_workspace) return GDPA_EINVAL;
  return fwd_impl(p, Q, K, V, nullptr, nullptr, nullptr, q_offsets, kv_offsets, bias, O, lse,
                  workspace, workspace_bytes, bwd_workspace, bwd_workspace_bytes, stream);
}

int32_t gdpa_fwd_static(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                        const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                        void* O, float* lse, void* stream) {
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (fwd_layout(p).total > GDPA_STATIC_SCRATCH_BYTES) return GDPA_EWORKSPACE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != GDPA_OK) return st;
  return gdpa_fwd(p, Q, K, V, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, O, lse, ws,
                  GDPA_STATIC_SCRATCH_BYTES, stream);
}

// The bias-gradient reduction of a backward call (both stages) on stream s.
static hipError_t launch_dbias(const gdpa_problem* p, const Prob& pr, const BwdArgs& ba, const SchedArgs& sq,
                               const int32_t* q_offsets, const int32_t* kv_offsets, float* dbias, char* ws,
                               const BwdLayout& L, int tq, hipStream_t s) {
  DbiasArgs da;
  da.q_off = q_offsets; da.kv_off = kv_offsets; da.tile_base = ba.tile_base;
  da.split_slot = sq.split_slot; da.part_x = ba.dbias_part_x;
  da.part = ba.dbias_part; da.part_rows = ba.part_rows; da.part_bh = (float*)(ws + L.part_bh); da.dbias = dbias;
  da.hdr = ws + L.header; da.B = p->B; da.H = p->H; da.nb = p->bias_buckets;
  da.causal = p->causal; da.win = pr.win; da.tile_rows = tq;
  da.loop_rows = bwd_k_loop(p->dtype);
  return launch_dbias_reduce(da, s);
}

// gdpa_bwd, or with planned the same on lists a gdpa_fwd_plan_bwd wrote (gdpa_bwd_planned).
static int32_t bwd_impl(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                        const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                        const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                        float* dbias, void* workspace, size_t workspace_bytes, bool planned,
                        void* stream) {
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (p->dtype == GDPA_MXFP8_E4M3) return GDPA_ENOTSUP;
  st = check_bwd_args(p, Q, K, V, O, dO, lse, q_offsets, kv_offsets, bias, dQ, dK, dV, dbias,
                      workspace);
  if (st != GDPA_OK) return st;
  const BwdLayout L = bwd_layout(p);
  if (workspace_bytes < L.total) return GDPA_EWORKSPACE;
  if (L.max_q_items > INT32_MAX || L.max_k_items > INT32_MAX) return GDPA_ENOTSUP;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const Prob pr = to_prob(p);
  const int tq = bwd_q_item(p->dtype);

  // query-tile and key-tile items, built in one launch (or already by gdpa_fwd_plan_bwd: then
  // only on the workspace it planned, for the same problem and offsets, once)
  if (planned && !plan_take(workspace, p, q_offsets, kv_offsets)) return GDPA_EINVAL;
  SchedArgs sq, sk;
  bwd_sched_args(p, pr, L, ws, q_offsets, kv_offsets, sq, sk);
  hipError_t e = hipSuccess;
  if (!planned) {
    plan_take(workspace, p, q_offsets, kv_offsets);  // the lists are rebuilt: any plan is gone
    e = launch_sched2(sq, sk, s);
    if (e != hipSuccess) return map_hip(e);
  }

  BwdArgs ba;
  ba.Q = Q; ba.K = K; ba.V = V; ba.O = O; ba.dO = dO; ba.lse = lse;
  ba.q_off = q_offsets; ba.kv_off = kv_offsets; ba.bias = bias;
  ba.dQ = dQ; ba.dK = dK; ba.dV = dV; ba.dbias = dbias;
  ba.Dvec = (float*)(ws + L.dvec); ba.hdr = ws + L.header;
  ba.items_q = ws + L.items_q; ba.items_k = ws + L.items_k;
  ba.dbias_part = p->bias_buckets > 0 ? (float*)(ws + L.part) : nullptr;
  ba.part_rows = (int)(L.max_qtiles * (tq / 32));
  ba.tile_base = (const int32_t*)(ws + L.tile_base);
  ba.dbias_part_x = (float*)(ws + L.part_x);
  ba.split_cnt_q = (int32_t*)(ws + L.split_cnt_q); ba.split_cnt_k = (int32_t*)(ws + L.split_cnt_k);
  ba.part_dq = (float*)(ws + L.part_dq); ba.part_dk = (float*)(ws + L.part_dk);
  ba.part_dv = (float*)(ws + L.part_dv);
  ba.H = p->H; ba.nb = p->bias_buckets; ba.scale = p->scale; ba.win = pr.win;
  ba.q_shared = p->q_shared;
  ba.dq_f32 = p->q_shared ? (float*)(ws + L.dq_f32) : nullptr;
  // The reductions that follow dQ (the shared seed block's dQ over samples, the bias gradient)
  // read only what dQ wrote, so for bf16 they run on a side stream beside dK/dV: their small
  // workgroups fit next to dK/dV's one per compute unit.
  auto reductions = [&](hipStream_t rs) -> hipError_t {
    hipError_t r = hipSuccess;
    if (p->q_shared) {
      DqSharedArgs qa;
      qa.q_off = q_offsets; qa.part = ba.dq_f32; qa.dQ = dQ; qa.hdr = ws + L.header;
      qa.B = p->B; qa.H = p->H; qa.D = p->D; qa.q_rows = pr.q_rows;
      qa.f32_out = p->dtype == GDPA_F32 ? 1 : 0;
      r = launch_dq_shared_reduce(qa, rs);
      if (r != hipSuccess) return r;
    }
    if (p->bias_buckets > 0) r = launch_dbias(p, pr, ba, sq, q_offsets, kv_offsets, dbias, ws, L, tq, rs);
    return r;
  };
  if (p->dtype != GDPA_F32 && (p->bias_buckets > 0 || p->q_shared)) {
    e = launch_bwd_bf16(pr, ba, (int)L.max_q_items, 0, s);
    if (e != hipSuccess) return map_hip(e);
    SideStream* side = side_stream();
    if (side != nullptr && (hipEventRecord(side->fork, s) != hipSuccess ||
                            hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess))
      return GDPA_EHIP;
    e = reductions(side != nullptr ? side->s : s);
    if (e != hipSuccess) return map_hip(e);
    if (side != nullptr && hipEventRecord(side->join, side->s) != hipSuccess) return GDPA_EHIP;
    e = launch_bwd_bf16(pr, ba, 0, (int)L.max_k_items, s);
    if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return GDPA_EHIP;
    return map_hip(e);
  }
  if (p->dtype == GDPA_F32) e = launch_bwd_f32(pr, ba, (int)L.max_q_items, (int)L.max_k_items, s);
  else e = launch_bwd_bf16(pr, ba, (int)L.max_q_items, (int)L.max_k_items, s);
  if (e != hipSuccess) return map_hip(e);
  return map_hip(reductions(s));
}

int32_t gdpa_bwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                 const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                 float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, Q, K, V, O, dO, lse, q_offsets, kv_offsets, bias, dQ, dK, dV, dbias,
                  workspace, workspace_bytes, false, stream);
}

int32_t gdpa_bwd_planned(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                         const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                         float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, Q, K, V, O, dO, lse, q_offsets, kv_offsets, bias, dQ, dK, dV, dbias,
                  workspace, workspace_bytes, true, stream);
}

int32_t gdpa_item_list(const gdpa_problem* p, int32_t for_bwd, int32_t list, size_t* offset,
                       int64_t* capacity) {
  if (!offset || !capacity) return GDPA_EINVAL;
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (for_bwd && p->dtype == GDPA_MXFP8_E4M3) return GDPA_ENOTSUP;
  if (list < 0 || list > (for_bwd ? 1 : 0)) return GDPA_EINVAL;
  if (!for_bwd) {
    const FwdLayout L = fwd_layout(p);
    *offset = L.items;
    *capacity = L.max_items;
  } else {
    const BwdLayout L = bwd_layout(p);
    *offset = list == 0 ? L.items_q : L.items_k;
    *capacity = list == 0 ? L.max_q_items : L.max_k_items;
  }
  return GDPA_OK;
}

namespace {

int32_t check_block_problem(const gdpa_block_problem* p) {
  if (p == nullptr) return GDPA_EINVAL;
  if (p->B < 0 || p->H < 1 || p->total < 0 || p->total >= (int64_t)1 << 31) return GDPA_EINVAL;
  if (p->dtype < GDPA_F32 || p->dtype > GDPA_MXFP8_E4M3) return GDPA_EINVAL;
  if (p->act < GDPA_ACT_SOFTMAX || p->act > GDPA_ACT_SILU) return GDPA_EINVAL;
  if (p->causal != 0 && p->causal != 1) return GDPA_EINVAL;
  if (p->rotary != 0 && p->rotary != 1) return GDPA_EINVAL;
  if (!isfinite(p->scale) || !isfinite(p->rope_base)) return GDPA_EINVAL;
  if (p->rotary && !(p->rope_base > 1.0f)) return GDPA_EINVAL;
  if (p->dtype != GDPA_BF16 || p->D != 128 || p->block != BLOCK_TOKENS) return GDPA_ENOTSUP;
  if (!(p->scale > 0.0f)) return GDPA_ENOTSUP;
  if ((int64_t)p->H * p->D > (1 << 20)) return GDPA_ENOTSUP;
  return GDPA_OK;
}

struct BlockLayout {
  size_t items, sched, total;
  int64_t max_items;
};

BlockLayout block_layout(const gdpa_block_problem* p) {
  BlockLayout L;
  L.max_items = items_bound(p->total, p->B, p->H, BLOCK_TOKENS, 0);
  L.items = ALIGN;
  L.sched = L.items + align_up((size_t)L.max_items * sizeof(Item));
  L.total = L.sched + align_up(sched_scratch_bytes(p->B, p->H));
  return L;
}

// Builds the item list (one per block and head), then runs the forward or backward kernel.
int32_t block_call(const gdpa_block_problem* p, const int32_t* offsets, BlockArgs& ba,
                   void* workspace, size_t workspace_bytes, void* stream, bool bwd) {
  const BlockLayout L = block_layout(p);
  if (workspace_bytes < L.total) return GDPA_EWORKSPACE;
  if (L.max_items > INT32_MAX) return GDPA_ENOTSUP;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  SchedArgs sa;
  sa.q_off = offsets; sa.kv_off = offsets; sa.B = p->B; sa.H = p->H;
  sa.total_q = p->total; sa.total_kv = p->total; sa.mode = SCHED_QTILES;
  sa.causal = 0; sa.win = 0; sa.q_rows = 0;
  sa.tile_item = BLOCK_TOKENS; sa.tile_loop = BLOCK_TOKENS;
  sa.max_items = (int)L.max_items; sa.list = 0; sa.split = 0; sa.nslot = SPLIT_NSLOT;
  sa.tile_base = nullptr; sa.split_slot = nullptr; sa.split_cnt = nullptr;
  sa.ws_header = ws; sa.items = ws + L.items;
  set_sched_scratch(sa, ws + L.sched, p->B);
  hipError_t e = launch_sched(sa, s);
  if (e != hipSuccess) return map_hip(e);
  ba.off = offsets; ba.hdr = ws; ba.items = ws + L.items; ba.H = p->H; ba.scale = p->scale;
  ba.rope_log2_base = p->rotary ? log2((double)p->rope_base) : 0.0;
  e = launch_block(p->act, p->causal != 0, p->rotary != 0, ba, (int)L.max_items, bwd, s);
  return map_hip(e);
}

}  // namespace

int32_t gdpa_block_workspace_size(const gdpa_block_problem* p, size_t* bytes) {
  if (bytes == nullptr) return GDPA_EINVAL;
  const int32_t st = check_block_problem(p);
  if (st != GDPA_OK) return st;
  *bytes = block_layout(p).total;
  return GDPA_OK;
}

int32_t gdpa_block_fwd(const gdpa_block_problem* p, const void* Q, const void* K, const void* V,
                       const int32_t* offsets, void* O, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const int32_t st = check_block_problem(p);
  if (st != GDPA_OK) return st;
  if (!offsets || !workspace) return GDPA_EINVAL;
  if (p->total > 0 && (!Q || !K || !V || !O)) return GDPA_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace) ||
      ((uintptr_t)offsets & 3u))
    return GDPA_EINVAL;
  BlockArgs ba = {};
  ba.Q = Q; ba.K = K; ba.V = V; ba.O = O;
  return block_call(p, offsets, ba, workspace, workspace_bytes, stream, false);
}

int32_t gdpa_block_bwd(const gdpa_block_problem* p, const void* Q, const void* K, const void* V,
                       const void* dO, const int32_t* offsets, void* dQ, void* dK, void* dV,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t st = check_block_problem(p);
  if (st != GDPA_OK) return st;
  if (!offsets || !workspace) return GDPA_EINVAL;
  if (p->total > 0 && (!Q || !K || !V || !dO || !dQ || !dK || !dV)) return GDPA_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || !aligned16(workspace) || ((uintptr_t)offsets & 3u))
    return GDPA_EINVAL;
  BlockArgs ba = {};
  ba.Q = Q; ba.K = K; ba.V = V; ba.dO = dO; ba.dQ = dQ; ba.dK = dK; ba.dV = dV;
  return block_call(p, offsets, ba, workspace, workspace_bytes, stream, true);
}

int32_t gdpa_bwd_mx(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                    const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                    const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                    const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                    float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (p->dtype != GDPA_MXFP8_E4M3) return GDPA_EINVAL;
  if (!workspace || !aligned16(workspace)) return GDPA_EINVAL;
  if ((p->total_q > 0 && (!Q || !q_scale)) || (p->total_kv > 0 && (!K || !V || !k_scale || !v_scale)))
    return GDPA_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V)) return GDPA_EINVAL;  // 16-byte code reads
  const MxBwdLayout L = mx_bwd_layout(p);
  if (workspace_bytes < L.total) return GDPA_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const gdpa_problem pb = bf16_view(p);
  // every argument is checked before anything is enqueued (the dequantised copies stand for Q,
  // K, V, and are 256-byte aligned workspace regions)
  st = check_problem(&pb);
  if (st != GDPA_OK) return st;
  st = check_bwd_args(&pb, ws + L.q, ws + L.k, ws + L.v, O, dO, lse, q_offsets, kv_offsets, bias,
                      dQ, dK, dV, dbias, ws + L.bwd);
  if (st != GDPA_OK) return st;
  {
    const BwdLayout LB = bwd_layout(&pb);
    if (LB.max_q_items > INT32_MAX || LB.max_k_items > INT32_MAX) return GDPA_ENOTSUP;
  }
  hipError_t e = launch_mx_dequant((const uint8_t*)Q, q_scale, ws + L.q, p->total_q, p->H, p->D, s);
  if (e == hipSuccess) e = launch_mx_dequant((const uint8_t*)K, k_scale, ws + L.k, p->total_kv, p->H, p->D, s);
  if (e == hipSuccess) e = launch_mx_dequant((const uint8_t*)V, v_scale, ws + L.v, p->total_kv, p->H, p->D, s);
  if (e != hipSuccess) return map_hip(e);
  return gdpa_bwd(&pb, ws + L.q, ws + L.k, ws + L.v, O, dO, lse, q_offsets, kv_offsets, bias, dQ,
                  dK, dV, dbias, ws + L.bwd, workspace_bytes - L.bwd, stream);
}

int32_t gdpa_read_device_error(const void* workspace, void* stream, int32_t* err) {
  if (!workspace || !err) return GDPA_EINVAL;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return GDPA_EHIP;
  WsHeader h;
  e = hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return GDPA_EHIP;
  *err = h.error;
  return GDPA_OK;
}

}  // extern "C"
