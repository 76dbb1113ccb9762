/*
 * gdpa.h - C ABI of libgdpa.so: attention over jagged (variable-length) sequences on MI355X.
 *
 * Two operations, forward and backward, for two families that share one structure, the product
 * Q.K^T (plus an optional bias), an element-wise map, and the product with V:
 *   - JFA: softmax attention computed directly on jagged tensors without padding (page "GEM
 *     Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", JFA
 *     paragraph: variable-length jagged tensors, custom attention biases, different query and
 *     key/value lengths, backward passes).
 *   - GDPA: the same two products with GELU (tanh form) or SiLU in place of softmax, and no
 *     normalisation (same page, GDPA paragraph: self-, PMA- and cross-attention as two matrix
 *     multiplications with an element-wise activation in between).
 *
 * Math, per sample b, head h, local query i in [0, Lq_b) and key j in [0, Lk_b):
 *   valid(i,j) = (!causal || j <= i) && (window == 0 || j > i - window)
 *   s_ij = scale * <q_i, k_j> + bias[h, clamp(i - j, 0, NB - 1)]   (no bias term if NB == 0)
 *   softmax: o_i = sum_j softmax_j(s_i.) v_j over valid j; lse_i = ln sum_j exp(s_ij)
 *            (a row with no valid key: o_i = 0, lse_i = -inf)
 *   GDPA:    o_i = sum_{valid j} act(s_ij) v_j
 *   gelu_tanh(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), silu(x) = x / (1 + e^-x)
 * The backward returns the gradients of sum(dO * O) with respect to Q, K, V and the bias table.
 *
 * Layout. A jagged tensor is a row-major array [total_rows, H, D] (D contiguous, row stride H*D
 * elements) plus int32 offsets[B + 1] (non-decreasing, offsets[0] = 0, offsets[B] = total_rows);
 * sample b owns rows [offsets[b], offsets[b+1]). Q, O, dO, dQ use q_offsets; K, V, dK, dV use
 * kv_offsets. lse is [total_q, H] fp32 (natural log). bias and dbias are [H, NB] fp32.
 * Element types: GDPA_F32 -> all tensors fp32; GDPA_BF16 -> Q/K/V/O/dO/dQ/dK/dV bf16;
 * GDPA_MXFP8_E4M3 (forward only) -> Q/K/V are e4m3 bytes with one e8m0 scale byte per 32
 * consecutive elements along D ([rows, H, D/32] arrays q_scale/k_scale/v_scale), O is bf16.
 * This MX encoding follows the OCP Microscaling Formats v1.0 (same page, low-precision part:
 * MXFP8 block-scaled matrix products).
 * Sliding-window attention (same page, the paragraph on sliding-window attention): with
 * causal = 1 and window = W >= 1, query i attends to keys i - W + 1 .. i only; on the bf16 path
 * tiles wholly outside the window are neither scheduled nor loaded.
 * Shared queries (PMA, same page, GDPA paragraph: a fixed set of learned seed queries attends to
 * every sample's keys): with q_shared = 1, Q and dQ are one block [max_q, H, D] used by every
 * sample, whose local query i reads row i; O, dO and lse stay jagged over q_offsets. The
 * backward returns dQ[i] = sum over samples b with Lq_b > i of the per-sample gradient, summed in
 * fp32 in a fixed order and rounded once.
 *
 * Ownership and synchronisation. Every pointer except `p` is device memory owned by the caller and
 * must stay valid until the work enqueued on `stream` (a hipStream_t; NULL = the null stream)
 * has finished. Calls are asynchronous: they validate host-side arguments, enqueue kernels and
 * return. The library allocates no device memory: scratch space comes from the caller's
 * `workspace`, whose size gdpa_workspace_size() returns from host-known sizes alone. Outputs are
 * overwritten, never accumulated. Base pointers must be 16-byte aligned.
 *
 * Errors. Host-checkable argument errors return a status and enqueue nothing. Data-dependent
 * errors (offsets not starting at 0, decreasing, or ending at a value other than total_q/total_kv;
 * with q_shared, a sample longer than max_q) are detected on the device: a device error word in the workspace is set, every kernel of the
 * call then skips its work and the outputs are left unspecified; gdpa_read_device_error() reads
 * that word. Nothing is printed and no C++ exception crosses this interface. Calls that share a
 * workspace must be ordered on one stream.
 */
#ifndef GDPA_H_
#define GDPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDPA_ACT_SOFTMAX = 0, GDPA_ACT_GELU_TANH = 1, GDPA_ACT_SILU = 2 } gdpa_act;

typedef enum { GDPA_F32 = 0, GDPA_BF16 = 1, GDPA_MXFP8_E4M3 = 2 } gdpa_dtype;

typedef enum {
  GDPA_OK = 0,
  GDPA_EINVAL = 1,     /* a null or misaligned pointer, a negative size, a bad enum value */
  GDPA_ENOTSUP = 2,    /* valid but unsupported: D not in {32, 64, 128}, MX in gdpa_bwd,
                          scale <= 0 outside fp32, a window on an MX problem, ... */
  GDPA_EWORKSPACE = 3, /* workspace_bytes smaller than gdpa_workspace_size() */
  GDPA_EHIP = 4        /* the HIP runtime refused a launch */
} gdpa_status;

/* Problem description; plain integers so the layout is stable across compilers. */
typedef struct {
  int32_t B;            /* samples (>= 0) */
  int32_t H;            /* heads (>= 1) */
  int32_t D;            /* head dimension: 32, 64 or 128 */
  int32_t dtype;        /* gdpa_dtype */
  int64_t total_q;      /* rows of Q/O/dO (= q_offsets[B]) */
  int64_t total_kv;     /* rows of K/V (= kv_offsets[B]) */
  int32_t max_q;        /* an upper bound on any Lq_b, or 0 if unknown; only tunes scheduling */
  int32_t max_kv;       /* an upper bound on any Lk_b, or 0 if unknown; only tunes scheduling */
  int32_t act;          /* gdpa_act */
  int32_t causal;       /* 0 or 1: keep j <= i on local positions (top-left aligned) */
  float scale;          /* s = scale * q.k (+ bias); must be > 0 for GDPA_BF16 / GDPA_MXFP8_E4M3 */
  int32_t bias_buckets; /* NB >= 0; 0 = no bias table */
  int32_t window;       /* W >= 0; 0 = no window. W >= 1 keeps keys j > i - W and needs causal = 1
                           and GDPA_F32 or GDPA_BF16 (otherwise GDPA_ENOTSUP). A W that no query
                           can reach (W >= total_q, or W >= max_q when max_q > 0) drops nothing and
                           is the same as no window; any other W >= 1 needs
                           total_q + total_kv <= INT32_MAX - 1024 (otherwise GDPA_ENOTSUP) */
  int32_t q_shared;     /* 0 or 1. 1: Q and dQ are [max_q, H, D], shared by all samples; needs
                           GDPA_BF16 or GDPA_F32 (else GDPA_ENOTSUP) and max_q >= 1 (else
                           GDPA_EINVAL); a
                           sample with Lq_b > max_q is a malformed q_offsets (device error 1) */
} gdpa_problem;

/* ABI version of this header (checked by bindings). */
#define GDPA_ABI_VERSION 3
int32_t gdpa_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* gdpa_status_string(int32_t status);

/* Bytes of device workspace that gdpa_fwd (for_bwd = 0) or gdpa_bwd (for_bwd = 1) needs for
 * problem *p. Depends only on the fields of *p. */
int32_t gdpa_workspace_size(const gdpa_problem* p, int32_t for_bwd, size_t* bytes);

/* Forward. Writes O ([total_q, H, D]) and, when lse != NULL, lse ([total_q, H]; softmax only, it
 * is what gdpa_bwd needs). q_scale/k_scale/v_scale are used only for GDPA_MXFP8_E4M3 and must be
 * NULL otherwise. bias is NULL iff p->bias_buckets == 0. */
int32_t gdpa_fwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                 const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                 const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias, void* O,
                 float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of sum(dO * O). Writes dQ, dK, dV (same layouts and element type as Q, K, V) and,
 * when p->bias_buckets > 0, dbias ([H, NB] fp32). Softmax needs O and the forward's lse; GDPA
 * ignores them (they may be NULL). Results are bitwise reproducible run to run. For bf16 with a
 * bias table or a shared query block, the reductions that follow dQ run on a second stream of the
 * library's (one per device and calling thread, default priority, created on first use and kept)
 * that waits on `stream` after dQ and that `stream` waits on before the call's last kernel
 * completes: to the caller all work stays ordered on `stream`, including under graph capture. */
int32_t gdpa_bwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                 const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                 float* dbias, void* workspace, size_t workspace_bytes, void* stream);

/* Forward of a training step that also schedules its backward (a step runs the forward and then
 * the backward on the same offsets; the scheduler, page "GEM Training: How Meta Doubled the
 * Efficiency of Its LLM-Scale Ads Foundation Model", JFA and GDPA paragraphs, is the same one).
 * Arguments and results as gdpa_fwd (bf16 and fp32 only: GDPA_ENOTSUP for GDPA_MXFP8_E4M3),
 * plus the backward's workspace (16-byte aligned, at least gdpa_workspace_size(p, 1, ...) bytes,
 * not overlapping the forward's, else GDPA_EINVAL / GDPA_EWORKSPACE): the forward's scheduler launch also builds the backward's
 * two work-item lists there, in workgroups of their own beside the forward's list, so that
 * gdpa_bwd_planned on that workspace needs no scheduler launch. Malformed offsets set the device
 * error word of both workspaces. */
int32_t gdpa_fwd_plan_bwd(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                          void* O, float* lse, void* workspace, size_t workspace_bytes,
                          void* bwd_workspace, size_t bwd_workspace_bytes, void* stream);

/* Backward on a workspace whose work-item lists gdpa_fwd_plan_bwd wrote. Arguments and results
 * as gdpa_bwd; the call must use the same problem *p and the same offsets (contents unchanged),
 * and be ordered after that gdpa_fwd_plan_bwd with no other call on the workspace in between:
 * one planned backward per plan (its kernels use up the lists' claim counters). The library
 * keeps, per workspace and device, a record of the last plan (problem fields and offset
 * pointers; gdpa_bwd on the workspace drops it): without a matching record the call returns
 * GDPA_EINVAL and enqueues nothing, and a matching record is used up. The offsets' contents are
 * not checked: lists planned for other offset values give unspecified results. */
int32_t gdpa_bwd_planned(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                         const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                         float* dbias, void* workspace, size_t workspace_bytes, void* stream);

/* Forward for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Same arguments and results as gdpa_fwd minus
 * the workspace. The scratch space gdpa_fwd takes from its workspace (work-item list, chunk
 * counters, partial results of split tiles) is instead one fixed buffer of
 * GDPA_STATIC_SCRATCH_BYTES inside the library, one per GPU, placed in device memory when the
 * library's code is loaded on that GPU and held until the process ends; the first call on a GPU
 * looks up its address there. No call allocates device memory. The GPU is the calling thread's
 * current device. A problem whose gdpa_workspace_size(p, 0, ...) exceeds
 * GDPA_STATIC_SCRATCH_BYTES returns GDPA_EWORKSPACE and enqueues nothing; other errors are those
 * of gdpa_fwd. Every call on one GPU uses that GPU's one buffer, which keeps the last call's
 * contents (nothing in it has to start at zero): calls that can overlap in time on one GPU
 * (different streams, different host threads) race on it and must be ordered by the caller, for
 * example on one stream. Its device error word cannot be read back; gdpa_fwd with a workspace
 * diagnoses malformed offsets. */
#define GDPA_STATIC_SCRATCH_BYTES ((size_t)48 << 20)
int32_t gdpa_fwd_static(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                        const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                        void* O, float* lse, void* stream);

/* Block-aligned attention with rotary embeddings (same page, block-attention paragraph): every
 * sample is cut into fixed blocks of `block` consecutive tokens (the last one shorter), and each
 * block attends only within itself, with the softmax or GDPA activation of the other entry points
 * and no bias table. With rotary = 1, Q and K are first rotated at their positions in the sample
 * (counted from its first token): the pair (2m, 2m+1) of a row at position p turns by
 * p * rope_base^(-2m/D) radians (the rotary form of Su et al.); the backward turns the gradients
 * of Q and K back (the transpose) in fp32. causal = 1 keeps key j <= query i inside a block.
 * A block fits one tile, so the kernels take the softmax's row maximum and sum in one pass and
 * form the backward's row term from P and dP in the tile: no logsumexp is written, and the
 * backward needs neither O nor lse.
 * Supported: GDPA_BF16, D = 128, block = 64, scale > 0 (else GDPA_ENOTSUP). Q, K, V, O, dO, dQ,
 * dK, dV are [total, H, 128] bf16 over one offsets array [B + 1]. Memory, workspace, stream and
 * error conventions are those of gdpa_fwd / gdpa_bwd; malformed offsets set device error 3
 * (the one offsets array is checked as both the query and the key offsets). */
typedef struct {
  int32_t B;         /* samples (>= 0) */
  int32_t H;         /* heads (>= 1) */
  int32_t D;         /* head dimension: 128 */
  int32_t dtype;     /* gdpa_dtype: GDPA_BF16 */
  int64_t total;     /* rows of every tensor (= offsets[B]) */
  int32_t act;       /* gdpa_act */
  int32_t causal;    /* 0 or 1: keep j <= i inside a block */
  float scale;       /* s = scale * q.k */
  int32_t block;     /* tokens per block: 64 */
  int32_t rotary;    /* 0 or 1 */
  float rope_base;   /* rotary base (> 1), e.g. 10000 */
} gdpa_block_problem;

int32_t gdpa_block_workspace_size(const gdpa_block_problem* p, size_t* bytes);
int32_t gdpa_block_fwd(const gdpa_block_problem* p, const void* Q, const void* K, const void* V,
                       const int32_t* offsets, void* O, void* workspace, size_t workspace_bytes,
                       void* stream);
/* Gradients of sum(dO * O) with respect to Q, K and V (bf16, overwritten). */
int32_t gdpa_block_bwd(const gdpa_block_problem* p, const void* Q, const void* K, const void* V,
                       const void* dO, const int32_t* offsets, void* dQ, void* dK, void* dV,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Backward for MX-fp8 inputs (GDPA_MXFP8_E4M3; same page, low-precision part: MXFP8 for the
 * forward and the backward). Arguments as gdpa_bwd plus the e8m0 scale arrays of Q, K and V
 * ([rows, H, D/32] u8, as for gdpa_fwd). Returns the gradients of sum(dO * O) with respect to the
 * dequantised values (the e4m3 code times its block's power of two), in bf16; O and lse come
 * from gdpa_fwd on the same inputs. Q, K and V are first dequantised exactly to bf16 in the
 * workspace (an e4m3 value times a power of two has at most 4 significant bits), so every
 * matrix product, the recomputed scores included, sees exactly the values the MX forward's
 * scaled products see; the gradient products then run as in the bf16 backward (their operands'
 * scales run along D, not along the contraction). gdpa_workspace_size(p, 1, ...) gives the
 * workspace. gdpa_bwd itself returns GDPA_ENOTSUP for MX problems. */
int32_t gdpa_bwd_mx(const gdpa_problem* p, const void* Q, const void* K, const void* V,
                    const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                    const void* O, const void* dO, const float* lse, const int32_t* q_offsets,
                    const int32_t* kv_offsets, const float* bias, void* dQ, void* dK, void* dV,
                    float* dbias, void* workspace, size_t workspace_bytes, void* stream);

/* Waits for `stream`, then reads the device error word of the last call that used `workspace`
 * (0 = none, 1 = malformed q_offsets, 2 = malformed kv_offsets). Diagnostics only. */
int32_t gdpa_read_device_error(const void* workspace, void* stream, int32_t* err);

/* Diagnostics (host-only, reads nothing from the device): where the scheduler's work-item list
 * `list` sits in a workspace of problem *p. The forward (for_bwd = 0) has list 0, its query-tile
 * items; the backward has list 0 (query-tile items, dQ) and list 1 (key-tile items, dK/dV).
 * *offset receives the list's byte offset from the start of the workspace and *capacity the
 * number of items it can hold; the workspace header's item counts (int32 words 1 and 2) say
 * how many items the last call wrote. An item is 12 int32: sample, tile, head, the tile's
 * canonical index (tiles numbered sample by sample), the first and one-past-last inner tile it
 * covers, its chunk slot (-1 when its tile is not split), chunk index | chunk count << 16, and
 * the sample's first query row, query length, first key row and key length.
 * Placement: item i runs on die i % 8 of the GPU. The (sample, head) groups are ranked by cost
 * (inner tiles, all of the group's items), largest first, and dealt to the dies in a snake
 * (0..7, 7..0, ...); each die lists its groups in rank order, a group's items consecutive with
 * its costliest tile first, and its q-th item takes index 8q + die. Header words 7..14 (list 0)
 * and 15..22 (list 1) hold each die's item count c_x. Die x takes indices 8q + x for
 * q < t_x = floor(n / 8) + (x < n mod 8 ? 1 : 0); a die with c_x > t_x passes its last items,
 * in order, to the dies with c_x < t_x (dies in increasing order, each from q = c_x on), so
 * the list of n items is dense. The D = 128 bf16 dQ and dK/dV kernels consume their list with one
 * workgroup per compute unit: workgroup i takes die (i mod 8)'s items in order of q by counting
 * on that die's claim counter, header words 23..30 (list 0) and 31..38 (list 1), which the
 * scheduler clears (after a call they hold counts past t_x; they are not item counts). The tiles
 * are those of the page named above, JFA paragraph: short sequences must not idle the GPU, so the
 * list balances and splits work by cost. */
int32_t gdpa_item_list(const gdpa_problem* p, int32_t for_bwd, int32_t list, size_t* offset,
                       int64_t* capacity);

/* Profiling aid for benchmarks. Between gdpa_profile_start(mask) and gdpa_profile_stop(), every
 * launch of a selected kernel is bracketed by a pair of HIP events recorded on its launch stream.
 * Launches stay reentrant while profiling is on (several host threads may launch; each launch
 * claims its own event pair), but gdpa_profile_start, _read and _stop must not run concurrently
 * with one another or with launches of the kernels they select. Bit k of mask selects kernel k: 0 = forward main kernel,
 * 1 = backward dQ kernel, 2 = backward dK/dV kernel, 3 = scheduler, 4 / 5 = block-aligned
 * forward / backward. At most 1024 launches per
 * kernel are timed. gdpa_profile_read() waits for the recorded events of one kernel and returns
 * how many of its launches were timed and their summed duration in milliseconds. Events are
 * created on the first start and kept for the life of the process. */
int32_t gdpa_profile_start(int32_t mask);
int32_t gdpa_profile_read(int32_t kernel, int32_t* launches, double* total_ms);
int32_t gdpa_profile_stop(void);

#ifdef __cplusplus
}
#endif

#endif /* GDPA_H_ */
