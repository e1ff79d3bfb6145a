// C ABI of the ragged extreme-GQA attention library (declared in
// include/attn_varlen.h): argument checks, workspace layout and the launch
// sequence of each entry point.  Everything is enqueued on the caller's
// stream; nothing here synchronises except attn_varlen_check_plan.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "attn_varlen.h"
#include "entry.hpp"
#include "kernels.hpp"

using namespace rga;

namespace {

thread_local std::string g_last_error;

attn_status vfail(attn_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_last_error = buf;
  return st;
}

attn_status fail(attn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

constexpr size_t ALIGN = 256;
constexpr int MAX_DEVICES = 64;
// Fixed cost of a dK/dV segment (K / V loads, the pipeline's unoverlapped
// first and last steps, the stores) in 64-row steps, for the work split; about
// 15 us against about 2.9 us per step, measured on the Hq = 64 workload.
constexpr int KV_SEGMENT_ITEMS = 5;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Compute-unit count per device, read once (the only state the library keeps).
int device_cus() {
  static int cache[MAX_DEVICES] = {0};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Layout {
  size_t seq, flag, zero, fwd_map, ktab, wg_first, kv_head, ksteps, head_hw;
  size_t lse, rowinfo, droprec, part_dk, part_dv;
  size_t total;
  int64_t kv_wgs;       // dK/dV workgroups (one per compute unit)
  int64_t row_tiles;
  int64_t kv_tiles;     // upper bound of the 128-key tiles
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dropout_on(const attn_problem* p) { return p->dropout_p > 0.0f || p->dropout_rates; }

Layout make_layout(const attn_problem* p, int entry, int cus) {
  Layout L{};
  // plan sequences: one per (packed sequence, K/V head)
  const int64_t B = (int64_t)p->batch * p->hkv;
  const int64_t rows = p->total_q * p->hq;
  L.row_tiles = ceil_div(rows, ROW_TILE) + B;
  L.kv_tiles = ceil_div(p->total_k * p->hkv, KEY_TILE) + B;
  L.kv_wgs = cus;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.flag = take(sizeof(int) * 4);   // first, so attn_varlen_check_plan can find it
  L.zero = take(512);
  L.seq = take(sizeof(int) * B * SEQ_FIELDS);
  L.fwd_map = take(sizeof(int) * 2 * (size_t)L.row_tiles);
  L.ktab = take(sizeof(int) * KV_FIELDS * (size_t)L.kv_tiles);
  L.wg_first = take(sizeof(int) * (size_t)L.kv_wgs);
  L.kv_head = take(sizeof(int) * 4);
  L.ksteps = take(sizeof(int) * 2 * (size_t)L.row_tiles);
  L.head_hw = take(sizeof(int) * (size_t)p->batch * p->hq);
  L.lse = L.rowinfo = L.droprec = L.part_dk = L.part_dv = 0;
  if (entry == ATTN_ENTRY_FULL_VJP) L.lse = take(sizeof(float) * rows);
  if (entry != ATTN_ENTRY_FWD) {
    L.rowinfo = take(sizeof(float) * 4 * rows);
    if (dropout_on(p)) L.droprec = take(sizeof(uint32_t) * 4 * rows);
    // FP32 partial dK / dV: two key tiles per workgroup (its first and last)
    const size_t part = sizeof(float) * 2 * (size_t)L.kv_wgs * KEY_TILE * p->head_dim;
    L.part_dk = take(part);
    L.part_dv = take(part);
  }
  L.total = off;
  return L;
}

attn_status check_problem(const attn_problem* p) {
  if (!p) return fail(ATTN_INVALID_ARG, "problem is NULL");
  if (p->dtype != ATTN_F16 && p->dtype != ATTN_BF16)
    return fail(ATTN_UNSUPPORTED, "dtype %d is neither F16 nor BF16", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 160)
    return fail(ATTN_UNSUPPORTED, "head_dim %d is not 64, 128 or 160", p->head_dim);
  if (p->causal != 0 && p->causal != 1)
    return fail(ATTN_INVALID_ARG, "causal must be 0 or 1 (got %d)", p->causal);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_INVALID_ARG, "window bounds must be >= -1 (got %d, %d)", p->window_left,
                p->window_right);
  if (p->batch < 0) return fail(ATTN_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->hq < 1 || p->hq > 1024) return fail(ATTN_INVALID_ARG, "hq %d outside 1..1024", p->hq);
  if (p->hkv < 1 || p->hq % p->hkv != 0)
    return fail(ATTN_INVALID_ARG, "hkv %d must be >= 1 and divide hq %d", p->hkv, p->hq);
  if ((int64_t)p->batch * p->hkv > (1 << 24))
    return fail(ATTN_INVALID_ARG, "batch x hkv %lld exceeds 2^24",
                (long long)p->batch * p->hkv);
  if (p->total_q < 0 || p->total_k < 0)
    return fail(ATTN_INVALID_ARG, "negative token count");
  if (p->total_q + p->total_k > INT32_MAX ||
      p->total_q * (int64_t)p->hq > (int64_t)INT32_MAX - 4 * ROW_TILE)
    return fail(ATTN_INVALID_ARG, "too many tokens for 32-bit row indices");
  if (!p->cu_q || !p->cu_k) return fail(ATTN_INVALID_ARG, "cu_q / cu_k is NULL");
  if (p->batch > 0 && !p->alibi_slopes) return fail(ATTN_INVALID_ARG, "alibi_slopes is NULL");
  if (p->slopes_stride < p->hq)
    return fail(ATTN_INVALID_ARG, "slopes_stride %lld < hq", (long long)p->slopes_stride);
  if (!(p->softcap >= 0.0f) || !std::isfinite(p->softcap))
    return fail(ATTN_INVALID_ARG, "softcap must be finite and >= 0");
  if (!std::isfinite(p->scale_multiplier))
    return fail(ATTN_INVALID_ARG, "scale_multiplier must be finite");
  if ((p->flags & ~ATTN_FLAG_ALL_KEYS) != 0)
    return fail(ATTN_INVALID_ARG, "unknown flags 0x%x", (unsigned)p->flags);
  if (!(p->dropout_p >= 0.0f && p->dropout_p < 1.0f))
    return fail(ATTN_INVALID_ARG, "dropout_p must lie in [0, 1)");
  return ATTN_OK;
}

attn_status check_tensor(const char* name, const attn_tensor* t, int64_t tokens, int heads,
                         int dim) {
  if (!t) return fail(ATTN_INVALID_ARG, "%s is NULL", name);
  if (tokens > 0 && !t->data) return fail(ATTN_INVALID_ARG, "%s.data is NULL", name);
  if (t->tok_stride < 0 || t->head_stride < 0)
    return fail(ATTN_INVALID_ARG, "%s has a negative stride", name);
  if (tokens > 1 && t->tok_stride < dim)
    return fail(ATTN_INVALID_ARG, "%s token stride %lld overlaps rows", name,
                (long long)t->tok_stride);
  if (heads > 1 && t->head_stride < dim)
    return fail(ATTN_INVALID_ARG, "%s head stride %lld overlaps rows", name,
                (long long)t->head_stride);
  if (t->tok_stride > INT32_MAX || t->head_stride > INT32_MAX)
    return fail(ATTN_INVALID_ARG, "%s strides must be below 2^31 elements", name);
  if ((reinterpret_cast<uintptr_t>(t->data) & 15) != 0 || (t->tok_stride & 7) != 0 ||
      (t->head_stride & 7) != 0)
    return fail(ATTN_MISALIGNED, "%s pointer or strides are not 16-byte multiples", name);
  return ATTN_OK;
}

LogitConsts logit_consts(const attn_problem* p) {
  LogitConsts lc;
  const double sigma = (double)p->scale_multiplier / std::sqrt((double)p->head_dim);
  const double l2e = 1.4426950408889634;
  const double c = p->softcap;
  lc.sigma = (float)sigma;
  lc.s_lin = (float)(sigma * l2e);
  if (c > 0) {
    lc.k_exp = (float)(2.0 * sigma * l2e / c);
    lc.t_mul = (float)(-2.0 * c * l2e);
    lc.t_add = (float)(c * l2e);
  } else {
    lc.k_exp = lc.t_mul = lc.t_add = 0.0f;
  }
  return lc;
}

Plan plan_view(void* ws, const Layout& L) {
  char* base = static_cast<char*>(ws);
  Plan pl;
  pl.seq = reinterpret_cast<int*>(base + L.seq);
  pl.ktab = reinterpret_cast<int*>(base + L.ktab);
  pl.wg_first = reinterpret_cast<int*>(base + L.wg_first);
  pl.kv_head = reinterpret_cast<int*>(base + L.kv_head);
  pl.flag = reinterpret_cast<int*>(base + L.flag);
  pl.fwd_map = reinterpret_cast<int*>(base + L.fwd_map);
  return pl;
}

attn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

#define RGA_TRY(expr)                          \
  do {                                         \
    const attn_status st__ = (expr);           \
    if (st__ != ATTN_OK) return st__;          \
  } while (0)

void set_view(const attn_tensor* t, const uint16_t** data, int64_t* ts, int64_t* hs) {
  *data = static_cast<const uint16_t*>(t->data);
  *ts = t->tok_stride;
  if (hs) *hs = t->head_stride;
}
void set_view(const attn_tensor* t, uint16_t** data, int64_t* ts, int64_t* hs) {
  *data = static_cast<uint16_t*>(t->data);
  *ts = t->tok_stride;
  if (hs) *hs = t->head_stride;
}

attn_status record(const hipEvent_t* ev, int i, hipStream_t s) {
  if (!ev) return ATTN_OK;
  return hip_status(hipEventRecord(ev[i], s), "event record");
}

// Shared prologue: checks and workspace.  Fills `a`, `L` and the planner's
// arguments `pa`; launches nothing.
attn_status prologue(const attn_problem* p, int entry, void* ws, size_t ws_bytes, AttnArgs& a,
                     Layout& L, PlanArgs& pa) {
  RGA_TRY(check_problem(p));
  const int cus = device_cus();
  L = make_layout(p, entry, cus);
  if (!ws && L.total > 0) return fail(ATTN_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < L.total)
    return fail(ATTN_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", ws_bytes, L.total);
  if ((reinterpret_cast<uintptr_t>(ws) & (ALIGN - 1)) != 0)
    return fail(ATTN_MISALIGNED, "workspace must be 256-byte aligned");
  std::memset(&a, 0, sizeof(a));
  a.slopes = p->alibi_slopes;
  a.slopes_stride = p->slopes_stride;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.group = p->hq / p->hkv;
  a.batch = p->batch * p->hkv;   // plan sequences
  a.total_q = p->total_q;
  a.total_k = p->total_k;
  a.lc = logit_consts(p);
  // far keys are skipped only under a cap (see row_key_steps)
  a.skip_log2 = 0.0f;
  if (p->softcap > 0.0f && (p->flags & ATTN_FLAG_ALL_KEYS) == 0)
    a.skip_log2 = (float)(SKIP_UNDERFLOW + 2.0 * p->softcap * 1.4426950408889634);
  a.plan = plan_view(ws, L);
  char* base = static_cast<char*>(ws);
  a.ksteps = reinterpret_cast<int*>(base + L.ksteps);
  a.zero = reinterpret_cast<const uint16_t*>(base + L.zero);
  if (L.rowinfo) a.rowinfo = reinterpret_cast<float*>(base + L.rowinfo);
  // dropout: the scalar rate's threshold floor(p 2^32) and scale, exact /
  // correctly rounded in double (the device derives per-row rates the same way)
  a.drop_on = dropout_on(p) ? 1 : 0;
  a.drop_seed = p->dropout_seed;
  a.drop_thr = (uint32_t)std::floor((double)p->dropout_p * 4294967296.0);
  a.drop_scale = (float)(1.0 / (1.0 - (double)p->dropout_p));
  a.drop_rates = p->dropout_rates;
  if (L.droprec) a.droprec = reinterpret_cast<u32x4*>(base + L.droprec);
  if (L.part_dk) {
    a.part_dk = reinterpret_cast<float*>(base + L.part_dk);
    a.part_dv = reinterpret_cast<float*>(base + L.part_dv);
  }
  std::memset(&pa, 0, sizeof(pa));
  pa.cu_q = p->cu_q;
  pa.cu_k = p->cu_k;
  pa.slopes = p->alibi_slopes;
  pa.slopes_stride = p->slopes_stride;
  pa.skip_log2 = a.skip_log2;
  pa.ksteps = a.ksteps;
  pa.head_hw = reinterpret_cast<int*>(base + L.head_hw);
  pa.batch = p->batch * p->hkv;
  pa.hq = p->hq / p->hkv;
  pa.hkv = p->hkv;
  pa.total_q = p->total_q;
  pa.total_k = p->total_k;
  pa.fwd_slots = (int)L.row_tiles;
  a.fwd_slots = (int)L.row_tiles;
  pa.kv_wgs = (int)L.kv_wgs;
  // A left bound of total_k or more keeps every key of every row (a row's
  // centre i + Lk - Lq is at most Lk - 1 < total_k), and so does a right bound
  // of total_q or more (the centre is at least Lk - Lq, so centre + total_q >=
  // Lk); clamping there keeps the kernels' bound arithmetic (centre -/+ bound)
  // inside int32, given total_q + total_k <= INT32_MAX.
  a.win_left = p->window_left < 0 ? -1 : (int)std::min<int64_t>(p->window_left, p->total_k);
  a.win_right = p->causal ? 0
                          : (p->window_right < 0 ? -1
                                                 : (int)std::min<int64_t>(p->window_right,
                                                                          p->total_q));
  // The forward ranks every row tile in LDS when the batch fits its limits
  // (the row-tile bound L.row_tiles over-counts the tiles, so a batch that
  // passes here always fits); otherwise it deals the tiles past its first
  // round by ticket, and the ticket is reset before each forward launch.
  const int64_t workers = std::max<int64_t>(1, L.kv_wgs - 1);
  const bool ranked = pa.batch <= LPT_MAX_SEQS &&
                      (int64_t)pa.batch * pa.hq <= LPT_MAX_HEADS &&
                      L.row_tiles <= LPT_MAX_TILES &&
                      ceil_div(L.row_tiles, workers) <= FWD_LIST_MAX;
  a.fwd_ticket = ranked ? nullptr : a.plan.flag + 2;
  pa.seg_items = KV_SEGMENT_ITEMS;
  pa.win_left = a.win_left;
  pa.win_right = a.win_right;
  a.kv_wgs = (int)L.kv_wgs;
  pa.zero = reinterpret_cast<uint16_t*>(base + L.zero);
  pa.plan = a.plan;
  // workspace past the fixed layout holds stored dS images (backward entries)
  pa.ds_images = 0;
  if (entry != ATTN_ENTRY_FWD && ws_bytes > L.total) {
    const size_t n = (ws_bytes - L.total) / DS_IMAGE_BYTES;
    pa.ds_images = (long long)std::min<size_t>(n, (size_t)INT32_MAX);
    if (pa.ds_images > 0) a.ds = reinterpret_cast<uint16_t*>(base + L.total);
  }
  return ATTN_OK;
}

// The planner as a launch of its own (after the views are set).
attn_status launch_prep_phase(const PlanArgs& pa, const AttnArgs& a, const Layout& L,
                              hipStream_t s, const hipEvent_t* ev = nullptr) {
  RGA_TRY(record(ev, ATTN_PHASE_PLAN, s));
  return hip_status(launch_prep(pa, s), "plan launch");
}

attn_status check_inputs(const attn_problem* p, const attn_tensor* q, const attn_tensor* k,
                         const attn_tensor* v) {
  RGA_TRY(check_tensor("q", q, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("k", k, p->total_k, p->hkv, p->head_dim));
  RGA_TRY(check_tensor("v", v, p->total_k, p->hkv, p->head_dim));
  return ATTN_OK;
}

// dK/dV, then dQ (which also sums the split dK/dV partials), after the row
// records are in place.
attn_status launch_backward(const attn_problem* p, const AttnArgs& a, const Layout& L,
                            hipStream_t s, const hipEvent_t* ev = nullptr) {
  const bool cap = p->softcap > 0.0f;
  if (p->batch > 0) {
    RGA_TRY(record(ev, ATTN_PHASE_DKDV, s));
    RGA_TRY(hip_status(launch_dkdv(a, p->dtype, p->head_dim, cap, (int)L.kv_wgs, s),
                       "dK/dV launch"));
    RGA_TRY(record(ev, ATTN_PHASE_DQ, s));
    // row tiles, then one partial-sum workgroup per compute unit
    RGA_TRY(hip_status(
        launch_dq(a, p->dtype, p->head_dim, cap, (int)L.row_tiles + device_cus(), s),
        "dQ launch"));
  }
  return ATTN_OK;
}

}  // namespace

namespace rga {

attn_status set_error(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error.clear(); }

attn_status full_vjp_impl(const attn_problem* p, const attn_tensor* q, const attn_tensor* k,
                          const attn_tensor* v, const attn_tensor* dout, const attn_tensor* out,
                          const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                          float* lse, void* workspace, size_t workspace_bytes, hipStream_t s,
                          const hipEvent_t* ev) {
  RGA_TRY(check_problem(p));
  RGA_TRY(check_inputs(p, q, k, v));
  RGA_TRY(check_tensor("dout", dout, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("out", out, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("dq", dq, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("dk", dk, p->total_k, p->hkv, p->head_dim));
  RGA_TRY(check_tensor("dv", dv, p->total_k, p->hkv, p->head_dim));
  AttnArgs a;
  Layout L;
  PlanArgs pa;
  RGA_TRY(prologue(p, ATTN_ENTRY_FULL_VJP, workspace, workspace_bytes, a, L, pa));
  set_view(q, &a.q, &a.q_ts, &a.q_hs);
  set_view(k, &a.k, &a.k_ts, &a.k_hs);
  set_view(v, &a.v, &a.v_ts, &a.v_hs);
  set_view(dout, &a.dout, &a.do_ts, &a.do_hs);
  set_view(out, &a.out, &a.o_ts, &a.o_hs);
  set_view(dq, &a.dq, &a.dq_ts, &a.dq_hs);
  set_view(dk, &a.dk, &a.dk_ts, &a.dk_hs);
  set_view(dv, &a.dv, &a.dv_ts, &a.dv_hs);
  a.lse = lse ? lse : reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse);
  // the planner runs inside the forward's grid (the plan phase is empty); an
  // empty batch runs the planner alone
  if (p->batch == 0) {
    RGA_TRY(launch_prep_phase(pa, a, L, s, ev));
    RGA_TRY(record(ev, ATTN_PHASE_FWD, s));
  } else {
    RGA_TRY(record(ev, ATTN_PHASE_PLAN, s));
    RGA_TRY(record(ev, ATTN_PHASE_FWD, s));
    if (a.fwd_ticket) RGA_TRY(hip_status(launch_ticket_reset(a.fwd_ticket, s), "ticket reset"));
    RGA_TRY(hip_status(launch_fwd(a, pa, p->dtype, p->head_dim, p->softcap > 0.0f, true, s),
                       "forward launch"));
  }
  RGA_TRY(launch_backward(p, a, L, s, ev));
  if (p->batch == 0) {
    RGA_TRY(record(ev, ATTN_PHASE_DKDV, s));
    RGA_TRY(record(ev, ATTN_PHASE_DQ, s));
  }
  return record(ev, ATTN_PHASES, s);
}

attn_status min_workspace(const attn_problem* p, int entry, size_t* bytes) {
  RGA_TRY(check_problem(p));
  *bytes = make_layout(p, entry, device_cus()).total;
  return ATTN_OK;
}

}  // namespace rga

extern "C" {

attn_status attn_varlen_workspace_size(const attn_problem* p, int entry, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(ATTN_INVALID_ARG, "bytes is NULL");
  RGA_TRY(check_problem(p));
  if (entry < ATTN_ENTRY_FWD || entry > ATTN_ENTRY_FULL_VJP)
    return fail(ATTN_INVALID_ARG, "unknown entry %d", entry);
  *bytes = make_layout(p, entry, device_cus()).total;
  return ATTN_OK;
}

attn_status attn_varlen_workspace_size_ds(const attn_problem* p, int entry,
                                          const int32_t* cu_q_host, const int32_t* cu_k_host,
                                          size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(ATTN_INVALID_ARG, "bytes is NULL");
  RGA_TRY(check_problem(p));
  if (entry < ATTN_ENTRY_FWD || entry > ATTN_ENTRY_FULL_VJP)
    return fail(ATTN_INVALID_ARG, "unknown entry %d", entry);
  if (!cu_q_host || !cu_k_host) return fail(ATTN_INVALID_ARG, "cu_q_host / cu_k_host is NULL");
  const int B = p->batch;
  if (cu_q_host[0] != 0 || cu_k_host[0] != 0 || cu_q_host[B] != p->total_q ||
      cu_k_host[B] != p->total_k)
    return fail(ATTN_BAD_SEQLENS, "cu_q / cu_k must start at 0 and end at total_q / total_k");
  size_t images = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t lq = (int64_t)cu_q_host[b + 1] - cu_q_host[b];
    const int64_t lk = (int64_t)cu_k_host[b + 1] - cu_k_host[b];
    if (lq < 0 || lk < 0) return fail(ATTN_BAD_SEQLENS, "cu_q / cu_k decrease at %d", b);
    if (lq > 0 && lk > 0)
      images += (size_t)p->hkv * (size_t)ceil_div(lq * (p->hq / p->hkv), ROW_TILE) *
                (size_t)ceil_div(lk, TILE_ROWS);
  }
  *bytes = make_layout(p, entry, device_cus()).total;
  if (entry != ATTN_ENTRY_FWD) *bytes += images * DS_IMAGE_BYTES;
  return ATTN_OK;
}

attn_status attn_varlen_fwd(const attn_problem* p, const attn_tensor* q, const attn_tensor* k,
                            const attn_tensor* v, const attn_tensor* out, float* lse,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  g_last_error.clear();
  RGA_TRY(check_problem(p));
  RGA_TRY(check_inputs(p, q, k, v));
  RGA_TRY(check_tensor("out", out, p->total_q, p->hq, p->head_dim));
  if (p->total_q > 0 && !lse) return fail(ATTN_INVALID_ARG, "lse is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs a;
  Layout L;
  PlanArgs pa;
  RGA_TRY(prologue(p, ATTN_ENTRY_FWD, workspace, workspace_bytes, a, L, pa));
  set_view(q, &a.q, &a.q_ts, &a.q_hs);
  set_view(k, &a.k, &a.k_ts, &a.k_hs);
  set_view(v, &a.v, &a.v_ts, &a.v_hs);
  set_view(out, &a.out, &a.o_ts, &a.o_hs);
  a.lse = lse;
  // an empty batch still runs the planner (it records the cu_q / cu_k check)
  if (p->batch == 0) return launch_prep_phase(pa, a, L, s);
  if (a.fwd_ticket) RGA_TRY(hip_status(launch_ticket_reset(a.fwd_ticket, s), "ticket reset"));
  return hip_status(launch_fwd(a, pa, p->dtype, p->head_dim, p->softcap > 0.0f, false, s),
                    "forward launch");
}

attn_status attn_varlen_bwd(const attn_problem* p, const attn_tensor* q, const attn_tensor* k,
                            const attn_tensor* v, const attn_tensor* out, const float* lse,
                            const attn_tensor* dout, const attn_tensor* dq,
                            const attn_tensor* dk, const attn_tensor* dv, void* workspace,
                            size_t workspace_bytes, attn_stream_t stream) {
  g_last_error.clear();
  RGA_TRY(check_problem(p));
  RGA_TRY(check_inputs(p, q, k, v));
  RGA_TRY(check_tensor("out", out, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("dout", dout, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("dq", dq, p->total_q, p->hq, p->head_dim));
  RGA_TRY(check_tensor("dk", dk, p->total_k, p->hkv, p->head_dim));
  RGA_TRY(check_tensor("dv", dv, p->total_k, p->hkv, p->head_dim));
  if (p->total_q > 0 && !lse) return fail(ATTN_INVALID_ARG, "lse is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs a;
  Layout L;
  PlanArgs pa;
  RGA_TRY(prologue(p, ATTN_ENTRY_BWD, workspace, workspace_bytes, a, L, pa));
  set_view(q, &a.q, &a.q_ts, &a.q_hs);
  set_view(k, &a.k, &a.k_ts, &a.k_hs);
  set_view(v, &a.v, &a.v_ts, &a.v_hs);
  a.out = static_cast<uint16_t*>(out->data);
  a.o_ts = out->tok_stride;
  a.o_hs = out->head_stride;
  set_view(dout, &a.dout, &a.do_ts, &a.do_hs);
  set_view(dq, &a.dq, &a.dq_ts, &a.dq_hs);
  set_view(dk, &a.dk, &a.dk_ts, &a.dk_hs);
  set_view(dv, &a.dv, &a.dv_ts, &a.dv_hs);
  a.lse = const_cast<float*>(lse);
  RGA_TRY(launch_prep_phase(pa, a, L, s));
  if (p->batch == 0) return ATTN_OK;
  RGA_TRY(hip_status(launch_rowinfo(a, p->dtype, p->head_dim, p->softcap > 0.0f, s), "row-record launch"));
  RGA_TRY(hip_status(launch_ksteps(a, (int)L.row_tiles, s), "key-step launch"));
  RGA_TRY(hip_status(launch_units(pa, s), "unit-plan launch"));
  return launch_backward(p, a, L, s);
}

attn_status attn_varlen_full_vjp_timed(const attn_problem* p, const attn_tensor* q,
                                       const attn_tensor* k, const attn_tensor* v,
                                       const attn_tensor* dout, const attn_tensor* out,
                                       const attn_tensor* dq, const attn_tensor* dk,
                                       const attn_tensor* dv, float* lse, void* workspace,
                                       size_t workspace_bytes, attn_stream_t stream,
                                       void* const* events) {
  g_last_error.clear();
  if (events) {
    for (int i = 0; i <= ATTN_PHASES; ++i)
      if (!events[i]) return fail(ATTN_INVALID_ARG, "events[%d] is NULL", i);
  }
  return full_vjp_impl(p, q, k, v, dout, out, dq, dk, dv, lse, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream),
                       reinterpret_cast<const hipEvent_t*>(events));
}

attn_status attn_varlen_full_vjp(const attn_problem* p, const attn_tensor* q,
                                 const attn_tensor* k, const attn_tensor* v,
                                 const attn_tensor* dout, const attn_tensor* out,
                                 const attn_tensor* dq, const attn_tensor* dk,
                                 const attn_tensor* dv, float* lse, void* workspace,
                                 size_t workspace_bytes, attn_stream_t stream) {
  return attn_varlen_full_vjp_timed(p, q, k, v, dout, out, dq, dk, dv, lse, workspace,
                                    workspace_bytes, stream, nullptr);
}

attn_status attn_varlen_check_plan(void* workspace, attn_stream_t stream) {
  g_last_error.clear();
  if (!workspace) return fail(ATTN_INVALID_ARG, "workspace is NULL");
  int flag = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RGA_TRY(hip_status(hipMemcpyAsync(&flag, workspace, sizeof(int), hipMemcpyDeviceToHost, s),
                     "reading the plan flag"));
  RGA_TRY(hip_status(hipStreamSynchronize(s), "stream synchronise"));
  if (flag != 0) return fail(ATTN_BAD_SEQLENS, "cu_q / cu_k are not a valid packing");
  return ATTN_OK;
}

attn_status attn_varlen_key_steps(const attn_problem* p, int entry, const void* workspace,
                                  int32_t* host_out, int64_t n_tiles, attn_stream_t stream) {
  g_last_error.clear();
  RGA_TRY(check_problem(p));
  if (entry < ATTN_ENTRY_FWD || entry > ATTN_ENTRY_FULL_VJP)
    return fail(ATTN_INVALID_ARG, "unknown entry %d", entry);
  if (!workspace) return fail(ATTN_INVALID_ARG, "workspace is NULL");
  const Layout L = make_layout(p, entry, device_cus());
  if (n_tiles < 0 || n_tiles > L.row_tiles)
    return fail(ATTN_INVALID_ARG, "n_tiles %lld outside 0..%lld", (long long)n_tiles,
                (long long)L.row_tiles);
  if (n_tiles == 0) return ATTN_OK;
  if (!host_out) return fail(ATTN_INVALID_ARG, "host_out is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* src = static_cast<const char*>(workspace) + L.ksteps;
  RGA_TRY(hip_status(hipMemcpyAsync(host_out, src, sizeof(int32_t) * 2 * (size_t)n_tiles,
                                    hipMemcpyDeviceToHost, s),
                     "reading the key steps"));
  return hip_status(hipStreamSynchronize(s), "stream synchronise");
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_INVALID_ARG: return "invalid argument";
    case ATTN_UNSUPPORTED: return "unsupported configuration";
    case ATTN_MISALIGNED: return "misaligned pointer or stride";
    case ATTN_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_HIP_ERROR: return "HIP runtime error";
    case ATTN_BAD_SEQLENS: return "cu_q / cu_k failed the device-side check";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
