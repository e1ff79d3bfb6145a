/*
 * attn_varlen.h -- C ABI of the MI355X (gfx950) ragged grouped-query attention
 * library: forward pass and full vector-Jacobian product.
 *
 * The operation (page "Noncausal Global Extreme-GQA Ragged Attention Full
 * VJP", sections "Hard Constraints" and "What You Have"):
 *
 *   For every sequence b of a packed ragged batch (query tokens
 *   [cu_q[b], cu_q[b+1]), key tokens [cu_k[b], cu_k[b+1])), every query head
 *   h and its K/V head g = h / (hq / hkv), with local positions i (query)
 *   and j (key),
 *   Lq = cu_q[b+1]-cu_q[b], Lk = cu_k[b+1]-cu_k[b], D = head_dim:
 *
 *     s_ij = (scale_multiplier / sqrt(D)) * <q_ih, k_jg>
 *     t_ij = softcap * tanh(s_ij / softcap)          (identity when softcap == 0)
 *     a_ij = t_ij - alibi_slopes[b, h] * |i + Lk - Lq - j|
 *     P_ij = softmax_j(a_ij) over the Lk keys of sequence b
 *     out_ih = sum_j P_ij v_jg,     lse_ih = log sum_j exp(a_ij)  (natural log)
 *
 *   The soft cap acts on the scaled dot product, before ALiBi.  The backward
 *   returns dq, dk, dv = the VJP of out against dout; dk and dv are summed over
 *   every query head that shares the K/V head.  Rows of a sequence with
 *   Lk == 0 get out = 0, dq = 0 and lse = -inf (page "python-20261012-ragged-
 *   flash-attention-gradient-recompute", section "Root causes addressed");
 *   keys of a sequence with Lq == 0 get dk = dv = 0.
 *
 * Masks.  The page's signature carries causal, window_left and window_right
 * but every case it defines is noncausal with no window (-1, -1).  Reading
 * taken for the other values: key j of local query row i is kept iff
 *   i + Lk - Lq - window_left <= j <= i + Lk - Lq + window_right,
 * a bound of -1 meaning no bound on that side and causal = 1 setting
 * window_right = 0 (aligned at the bottom right, like the ALiBi centre).  The
 * cap and ALiBi of kept keys are unchanged; a row that keeps no key is a row
 * with no keys (out = 0, dq = 0, lse = -inf).
 *
 * Dropout.  Page "python-20261012-ragged-flash-attention-gradient-recompute",
 * section "Root causes addressed": a counter-based splitmix64 hash of (seed,
 * b, h, row, col), so the backward rebuilds the forward's mask whatever the
 * tiling; one rate or one per row.  Reading taken: the (sequence b, query
 * head h) stream state is output b * 2^16 + h + 1 of splitmix64 (Steele, Lea
 * and Flood 2014) started at dropout_seed; the word of local row i and local
 * key j is output i * 2^32 + j + 1 of that stream; key j is kept iff the
 * word's top 32 bits reach floor(p * 2^32), and kept weights P_ij are scaled
 * by 1 / (1 - p).  Dropout acts after the softmax: lse is that of the
 * undropped weights, out = (P * mask / (1 - p)) V, and the backward is its
 * exact VJP.  Dropout is on when dropout_p > 0 or dropout_rates is not NULL;
 * per-row rates are read on the device and clamped to [0, 1 - 2^-24].
 *
 * Supported: dtype F16 or BF16 (one dtype for every 16-bit tensor), any hkv
 * dividing hq (grouped key/value heads), head_dim 64, 128 or 160 (page
 * "Pairwise-Gated Attention Engine", section "The task", names head sizes 64
 * and 128 and grouped K/V heads; the first page's cases are 160 over one K/V
 * head).  Another dtype or head_dim returns ATTN_UNSUPPORTED; hkv not
 * dividing hq, causal outside {0, 1} or a window bound below -1 returns
 * ATTN_INVALID_ARG.
 *
 * Tensors.  Every activation tensor is a strided view [tokens, heads, head_dim]
 * with a contiguous feature axis (feature stride 1) and caller-chosen token
 * and head strides, in elements.  Device pointers and both strides must be
 * multiples of 16 bytes / 8 elements (ATTN_MISALIGNED otherwise).  Offsets are
 * computed in 64-bit, so views may span more than 2^31 elements.
 *
 * Ownership and threading.  The caller allocates and owns every buffer,
 * including the workspace, whose size comes from attn_varlen_workspace_size.
 * The library allocates no device memory, never writes its inputs (padding
 * included) and keeps no state between calls except a per-device cache of the
 * compute-unit count.  Outputs must not alias inputs.  All work is enqueued
 * asynchronously on `stream`; nothing synchronises the host.  Calls on
 * different streams need different workspaces.
 *
 * Determinism.  No atomics are used; every reduction runs in a fixed order, so
 * repeated calls with identical inputs give bitwise-identical outputs.
 *
 * Far keys.  With softcap > 0 every capped logit lies in [-softcap, softcap],
 * so a key whose ALiBi term slope * |i + Lk - Lq - j| exceeds the row's largest
 * possible logit by enough (about 111 + 2 softcap in natural-log units) gets
 * P == 0 exactly in FP32, in the forward and in the backward.  The kernels
 * skip the 64-key steps in which every key is that far from every row of a
 * 256-row tile.  out, lse and dq are bitwise those of evaluating them, and dk
 * and dv agree to within rounding of the FP32 partial sums (the split of a key
 * tile's rows over workgroups follows the rows that visit it), provided the
 * skipped q / k / v / dout values are finite (non-finite values there are not
 * read, so they do not propagate).  ATTN_FLAG_ALL_KEYS turns this off.
 *
 * Errors.  Functions return an attn_status; a failed host-side check launches
 * nothing.  attn_last_error() gives a human-readable detail for the calling
 * thread.  Inconsistent cu_q / cu_k contents (not monotone, cu[0] != 0,
 * cu[B] != total) can only be seen on the device: the plan clamps them to
 * empty sequences and raises a flag that attn_varlen_check_plan() reads
 * (that call synchronises the stream).
 */
#ifndef RAGGED_GQA_ATTN_VARLEN_H
#define RAGGED_GQA_ATTN_VARLEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_INVALID_ARG = -1,          /* null pointer, bad size, feature stride != 1 */
  ATTN_UNSUPPORTED = -2,          /* head_dim or dtype outside the supported set */
  ATTN_MISALIGNED = -3,           /* pointer or stride not a multiple of 16 B */
  ATTN_WORKSPACE_TOO_SMALL = -4,
  ATTN_HIP_ERROR = -5,            /* a HIP runtime call or launch failed */
  ATTN_BAD_SEQLENS = -6           /* device-side cu_q / cu_k check failed */
} attn_status;

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Bits of attn_problem.flags. */
typedef enum {
  ATTN_FLAG_ALL_KEYS = 1   /* evaluate every key, also where P is exactly 0 */
} attn_flag;

typedef enum {
  ATTN_ENTRY_FWD = 0,
  ATTN_ENTRY_BWD = 1,
  ATTN_ENTRY_FULL_VJP = 2
} attn_entry;

/* A hipStream_t; NULL is the default stream. */
typedef void* attn_stream_t;

/* Strided view [tokens, heads, head_dim] of 16-bit elements, feature stride 1
 * (q, dout, out, dq: hq heads; k, v, dk, dv: hkv heads). */
typedef struct {
  void* data;            /* device pointer to element [0, 0, 0] */
  int64_t tok_stride;    /* elements between consecutive tokens */
  int64_t head_stride;   /* elements between consecutive heads */
} attn_tensor;

typedef struct {
  int32_t dtype;               /* attn_dtype */
  int32_t batch;               /* B >= 0 sequences */
  int32_t hq;                  /* query heads, 1..1024 */
  int32_t hkv;                 /* K/V heads, dividing hq; query head h reads head h / (hq / hkv) */
  int32_t head_dim;            /* 64, 128 or 160 */
  int64_t total_q;             /* tokens in the q / dout / out / dq views (= cu_q[B]) */
  int64_t total_k;             /* tokens in the k / v / dk / dv views (= cu_k[B]) */
  const int32_t* cu_q;         /* device int32 [B+1], cu_q[0] = 0, nondecreasing */
  const int32_t* cu_k;         /* device int32 [B+1] */
  const float* alibi_slopes;   /* device float32 [B, hq], row stride slopes_stride */
  int64_t slopes_stride;       /* elements between consecutive sequences (>= hq) */
  int32_t causal;              /* 0 or 1 (1: window_right is taken as 0) */
  int32_t window_left;         /* keys kept down to centre - window_left; -1 = all */
  int32_t window_right;        /* keys kept up to centre + window_right; -1 = all */
  float softcap;               /* c > 0 caps logits at c*tanh(x/c); 0 = no cap */
  float scale_multiplier;      /* logit scale = scale_multiplier / sqrt(head_dim) */
  int32_t flags;               /* attn_flag bits; 0 for the default behaviour */
  float dropout_p;             /* dropout rate in [0, 1); 0 = none (see "Dropout") */
  uint64_t dropout_seed;       /* seed of the counter-based dropout hash */
  const float* dropout_rates;  /* NULL, or device float32 [total_q, hq] contiguous per-row
                                  rates in [0, 1) that replace dropout_p */
} attn_problem;

/* Bytes of workspace that `entry` (attn_entry) needs for problem `p`.
 * Depends only on host-visible sizes (batch, hq, total_q, total_k). */
attn_status attn_varlen_workspace_size(const attn_problem* p, int entry, size_t* bytes);

/* Workspace with room for the stored dS of every sequence.
 *
 * The backward entries (ATTN_ENTRY_BWD, ATTN_ENTRY_FULL_VJP) use any workspace
 * bytes beyond attn_varlen_workspace_size to keep dS = P * (dP - Delta) *
 * (1 - tanh^2) in the input dtype, as the dK/dV pass forms it, so that dQ is
 * one product dS K instead of a second recomputation of S, P and dP (page
 * "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section "Hard
 * Constraints": the cap derivative multiplies dP - Delta).  A sequence needs
 * hkv * ceil(Lq * (hq / hkv) / 256) * ceil(Lk / 64) images of 32 KiB; sequences
 * (each K/V head in turn) get room in
 * batch order while it lasts and the rest recompute, so every workspace size
 * from the minimum up gives the same results to within rounding (the stored
 * and the recomputed dS round the same value; a sequence's dQ is bitwise
 * repeatable for a fixed workspace size).
 *
 * This function returns the size at which every sequence is stored, from host
 * copies of cu_q / cu_k (int32 [batch + 1], the same contents the device
 * arrays will hold).  Errors: ATTN_BAD_SEQLENS when they do not start at 0,
 * end at total_q / total_k and never decrease.  For ATTN_ENTRY_FWD it equals
 * attn_varlen_workspace_size. */
attn_status attn_varlen_workspace_size_ds(const attn_problem* p, int entry,
                                          const int32_t* cu_q_host, const int32_t* cu_k_host,
                                          size_t* bytes);

/* Forward: writes out (strided, dtype of q) and lse (float32 [total_q, hq]
 * contiguous, natural log, -inf for rows whose sequence has no keys). */
attn_status attn_varlen_fwd(const attn_problem* p,
                            const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_tensor* out, float* lse,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* Backward from a stored forward: given out and lse from attn_varlen_fwd and
 * the cotangent dout, writes dq (like q), dk and dv (like k / v). */
attn_status attn_varlen_bwd(const attn_problem* p,
                            const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                            const attn_tensor* out, const float* lse, const attn_tensor* dout,
                            const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* Forward plus full VJP in one call: writes out, dq, dk, dv; lse is written
 * when non-NULL (float32 [total_q, hq]) and kept in the workspace otherwise. */
attn_status attn_varlen_full_vjp(const attn_problem* p,
                                 const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                 const attn_tensor* dout,
                                 const attn_tensor* out, const attn_tensor* dq,
                                 const attn_tensor* dk, const attn_tensor* dv, float* lse,
                                 void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* Phases of attn_varlen_full_vjp, in launch order. */
typedef enum {
  ATTN_PHASE_PLAN = 0,     /* separate planning launch: only for an empty batch (the
                              planner otherwise runs inside the forward's grid) */
  ATTN_PHASE_FWD = 1,      /* forward: out, lse, delta = rowsum(dout * out); its first
                              workgroup plans the work lists from cu_q / cu_k */
  ATTN_PHASE_DKDV = 2,     /* dK, dV over all sharing heads */
  ATTN_PHASE_DQ = 3,       /* dQ, and the fixed-order sum of split dK / dV partials */
  ATTN_PHASES = 4
} attn_phase;

/* attn_varlen_full_vjp with per-phase timing.  `events` is NULL or holds
 * ATTN_PHASES + 1 hipEvent_t handles created by the caller; event i is
 * recorded on `stream` right before phase i is enqueued and event
 * ATTN_PHASES after the last one, so the elapsed time between events i and
 * i + 1 is phase i.  The computation is identical to attn_varlen_full_vjp. */
attn_status attn_varlen_full_vjp_timed(const attn_problem* p,
                                       const attn_tensor* q, const attn_tensor* k,
                                       const attn_tensor* v, const attn_tensor* dout,
                                       const attn_tensor* out, const attn_tensor* dq,
                                       const attn_tensor* dk, const attn_tensor* dv, float* lse,
                                       void* workspace, size_t workspace_bytes,
                                       attn_stream_t stream, void* const* events);

/* Bytes of the static scratch array of attn_varlen_full_vjp_noalloc (256 MiB
 * per GPU, 0.09 % of an MI355X's 288 GB). */
#define ATTN_NOALLOC_SCRATCH_BYTES (256u << 20)

/* attn_varlen_full_vjp for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid allocation):
 * it takes no workspace and allocates nothing.  Its workspace is a static
 * device array of ATTN_NOALLOC_SCRATCH_BYTES bytes that each GPU the library
 * runs on holds until the process ends; results are those of
 * attn_varlen_full_vjp with a workspace of that size (dS images in what the
 * minimum layout leaves free).  The caller still passes every input and
 * output.  Errors: those of attn_varlen_full_vjp, and ATTN_WORKSPACE_TOO_SMALL
 * when the problem's minimum workspace (attn_varlen_workspace_size) exceeds
 * the array.  All calls on one GPU share that GPU's array: calls that overlap
 * on one GPU (several streams or threads) race and must be ordered by the
 * caller; the device-side cu_q / cu_k check has no workspace to read back. */
attn_status attn_varlen_full_vjp_noalloc(const attn_problem* p,
                                         const attn_tensor* q, const attn_tensor* k,
                                         const attn_tensor* v, const attn_tensor* dout,
                                         const attn_tensor* out, const attn_tensor* dq,
                                         const attn_tensor* dk, const attn_tensor* dv,
                                         float* lse, attn_stream_t stream);

/* Synchronises `stream` and reports the device-side cu_q / cu_k check of the
 * last call that used `workspace`: ATTN_OK or ATTN_BAD_SEQLENS. */
attn_status attn_varlen_check_plan(void* workspace, attn_stream_t stream);

/* Diagnostics: the key steps the last call of `entry` on `workspace` (same
 * problem sizes) evaluated.  The folded rows of sequence b and K/V head g (row
 * h * Lq + i for local head h of g's group, token i) form
 * ceil(Lq * (hq / hkv) / 256) tiles of 256; for each tile, in batch order and
 * K/V head order inside a sequence, host_out receives two int32: the first
 * and one past the last 64-key step of the sequence that the tile's rows
 * visit (see "Far keys" above; 0 and ceil(Lk / 64) when nothing is skipped).
 * n_tiles is the number of such tiles (sum over b and g); host_out holds
 * 2 * n_tiles values.  Synchronises
 * `stream`.  Errors: ATTN_INVALID_ARG for a NULL pointer or n_tiles outside
 * 0 .. the bound the workspace layout allows; ATTN_HIP_ERROR if the copy
 * fails. */
attn_status attn_varlen_key_steps(const attn_problem* p, int entry, const void* workspace,
                                  int32_t* host_out, int64_t n_tiles, attn_stream_t stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RAGGED_GQA_ATTN_VARLEN_H */
