// Host-visible launchers of the gfx950 kernels and the argument block they share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace rga {

// Row-tile kernels (forward, dQ): one workgroup = 8 waves x 32 folded rows,
// two waves per SIMD so one wave's VALU work overlaps the other's MFMA.
constexpr int ROW_WAVES = 8;
constexpr int ROW_THREADS = ROW_WAVES * 64;
constexpr int ROW_TILE = ROW_WAVES * 32;
// Key-tile kernel (dK/dV): one workgroup = 8 waves = 4 wave pairs x 32 keys.
constexpr int KV_THREADS = 512;
constexpr int KEY_TILE = 128;
// Rows or keys of one LDS row tile (see tiles.hpp): the key step of the
// row-tile kernels and the row step of dK/dV.
constexpr int TILE_ROWS = 64;
// 16-bit elements of one row tile of head dimension D
template <int D> constexpr int tile_elems() { return TILE_ROWS * D; }
// Folded rows staged per step of the dK/dV kernel (each wave of a pair forms
// P and dS for half of them).
constexpr int KV_ROW_STEP = TILE_ROWS;
// Stored dS: one image per (row tile of ROW_TILE folded rows, 64-key step),
// 64 keys x ROW_TILE rows of 16-bit values (layout: ds_off in tiles.hpp).
constexpr int DS_IMAGE_ELEMS = TILE_ROWS * ROW_TILE;
constexpr size_t DS_IMAGE_BYTES = sizeof(uint16_t) * DS_IMAGE_ELEMS;

struct AttnArgs {
  const uint16_t* q;    int64_t q_ts, q_hs;
  const uint16_t* k;    int64_t k_ts;
  const uint16_t* v;    int64_t v_ts;
  const uint16_t* dout; int64_t do_ts, do_hs;
  uint16_t* out;        int64_t o_ts, o_hs;
  uint16_t* dq;         int64_t dq_ts, dq_hs;
  uint16_t* dk;         int64_t dk_ts;
  uint16_t* dv;         int64_t dv_ts;
  float* lse;           // [total_q * hq], natural log
  // [total_q * hq] records of 4 floats, one per folded row (sequence b's rows
  // at q0(b) * hq + R, R = h * Lq + i), read by the backward:
  //   slope * log2(e), the ALiBi centre i + Lk - Lq (clamped at 0, the centre
  //   the bias measures from, unless a window or causal mask is set: then
  //   unclamped, for the window test, and each reader clamps it),
  //   minus the base-2 log of the row's softmax sum relative to the row offset
  //   m_i (see fwd.hip), and Delta = rowsum(dout * out).
  float* rowinfo;
  const uint16_t* zero; // 512 zero bytes: source of the loads of rows past a tile's end
  float* part_dk;       // [units][KEY_TILE][D] FP32 partials (split sequences)
  float* part_dv;
  // dS images written by dK/dV and read by dQ for the sequences the planner
  // gave a slot (SQ_DSOFF >= 0); sequence images are row-tile major:
  // image SQ_DSOFF + row_tile * ceil(Lk / 64) + key_step.
  uint16_t* ds;
  // Key steps [lo, hi) (64 keys each) of every 256-row tile, batch order
  // (tile SQ_RTOFF + t of sequence b): the steps that hold a key whose P can
  // be nonzero for some row of the tile (see row_key_steps).  Written by the
  // planner (rewritten by ksteps_kernel in the standalone backward) and read
  // by the forward, dK/dV and dQ kernels.
  int* ksteps;
  // The forward's tile ticket (plan.flag[2]), reset to 0 by a launch just
  // before the forward; null when the forward deals every tile in its fixed
  // snake (the batches whose ranking fits a workgroup).  See fwd_kernel.
  int* fwd_ticket;
  // Skip bound in log2 units (0 turns skipping off): keys whose ALiBi term
  // slope * log2(e) * |c_i - j| exceeds it are dropped (the planner's ranges).
  float skip_log2;
  const float* slopes;  int64_t slopes_stride;
  int64_t k_hs, v_hs, dk_hs, dv_hs;   // K/V head strides (hkv > 1)
  int hq;               // query heads (row stride of lse and of the row records)
  int group;            // query heads per K/V head: the rows folded per plan sequence
  int hkv;
  int batch;            // plan sequences: packed sequences x hkv
  int64_t total_q;
  int64_t total_k;
  int fwd_slots;        // entries of plan.fwd_map; the dQ grid has more (partial sums)
  int kv_wgs;           // dK/dV workgroups (each takes an equal share of the visits)
  LogitConsts lc;
  Plan plan;
  // Key window of row i (local positions): keys j with
  // i + Lk - Lq - win_left <= j <= i + Lk - Lq + win_right are kept, a negative
  // bound being no bound (causal: win_right = 0); both negative = no mask.
  int win_left;
  int win_right;
  // Dropout (see dropout.hpp): the seed, the scalar rate's threshold and
  // scale, optional per-row rates [total_q, hq] (NULL: the scalar rate), and
  // the per-row records [total_q * hq] the backward reads (row record index).
  int drop_on;          // dropout with the fields below
  uint64_t drop_seed;
  uint32_t drop_thr;
  float drop_scale;
  const float* drop_rates;
  u32x4* droprec;
};

struct PlanArgs {
  const int* cu_q;
  const int* cu_k;
  const float* slopes;  int64_t slopes_stride;
  int batch;            // plan sequences (packed sequences x hkv)
  int hq;               // query heads per plan sequence (the group)
  int hkv;              // K/V heads: plan sequence v is packed sequence v / hkv
  int64_t total_q;
  int64_t total_k;
  // Skip bound of the key-step ranges the planner records (log2 units, 0 =
  // every key; see row_key_steps).
  float skip_log2;
  int* ksteps;          // [row tiles * 2] ranges the planner writes (AttnArgs::ksteps)
  int* head_hw;         // [B * hq] key half-widths, when they do not fit the planner's LDS
  int win_left;         // key window (AttnArgs::win_left / win_right): the ranges
  int win_right;        //   keep only the steps that hold some row's window keys
  long long ds_images;  // dS images that fit the workspace (0: no stored dS)
  int fwd_slots;        // entries of plan.fwd_map (the row-tile launches' grid)
  int kv_wgs;           // dK/dV workgroups (the dK/dV launch's grid)
  int seg_items;        // modelled fixed cost of a dK/dV segment, in 64-row steps
  uint16_t* zero;       // 512 bytes the planner clears
  Plan plan;
};


enum { DT_F16 = 0, DT_BF16 = 1 };

// Exact skipping of far keys (capped logits only).  With a cap c every scaled,
// capped logit of row i lies in [-c, c], so relative to the row offset the
// forward uses (the largest value any logit of the row can take, see fwd.hip)
// a key's exponent in log2 units is at most -slope2 |c_i - j| (slope2 =
// slope * log2 e, c_i the clamped ALiBi centre).  The backward adds the
// row's residual -log2 l, and l >= P of the centre key >= 2^(-2 c log2 e).
// Once the exponent is below -SKIP_UNDERFLOW, exp2 returns exactly 0 (FP32's
// smallest subnormal is 2^-149), so such a key adds exactly nothing to O, l,
// dQ, dK or dV: a key whose slope2 |c_i - j| exceeds
//   forward:  SKIP_UNDERFLOW + 2 c log2 e,
//   backward: SKIP_UNDERFLOW + max(0, residual of the row)
// is never evaluated: it would contribute exact zeros.
constexpr float SKIP_UNDERFLOW = 160.0f;

// Key steps [lo, hi) (64 keys) holding every key of one row that the bound
// `thr` (log2 units, 0 = none) keeps: the keys j with |c - j| <= floor(thr /
// slope2).  A row that does not exist gives the empty range (INT_MAX, 0), the
// neutral element of the min / max over a tile; rows whose slope is not a
// positive finite number, or whose kept span reaches the sequence's ends,
// keep every step.
// Half-width ds = floor(thr / slope2) of the keys a row keeps, or -1 when it
// keeps every key (no bound, a slope that is not a positive finite number, or
// a span that reaches past Lk).  A key outside [centre - ds, centre + ds] has
// |c - j| >= ds + 1 > thr / slope2.
__device__ __forceinline__ int key_half_width(float slope2, int Lk, float thr) {
  if (thr > 0.0f && slope2 > 0.0f) {   // false for NaN
    const float span = thr / slope2;   // +inf for a tiny slope
    if (span < (float)Lk) return (int)span;
  }
  return -1;
}

// Key steps of a row with the given centre and half-width (key_half_width).
__device__ __forceinline__ void key_steps_of(int centre, int ds, int Lk, int& lo, int& hi) {
  if (ds < 0) {
    lo = 0;
    hi = (Lk + TILE_ROWS - 1) / TILE_ROWS;
  } else {
    lo = max(0, centre - ds) / TILE_ROWS;
    hi = min(Lk - 1, centre + ds) / TILE_ROWS + 1;
  }
}

// A tile's final key-step range: (0, 0) when its rows keep no key (the
// per-row neutral element (INT_MAX, 0) never leaves a range computation), so
// every consumer sees lo <= hi and hi - lo >= 0.
__device__ __forceinline__ void finish_range(int& lo, int& hi) {
  if (lo >= hi) {
    lo = 0;
    hi = 0;
  }
}

// Key steps of query tokens [ia, ib] of a sequence: those of the ALiBi rule
// for the head's half-width ds (key_steps_of at the tokens' clamped centres,
// both bounds grow with the token), intersected with the key steps that hold
// some token's window keys [i + Lk - Lq - wl, i + Lk - Lq + wr] (a negative
// bound is no bound).  An empty result is lo >= hi.
__device__ __forceinline__ void token_range_steps(int ia, int ib, int Lq, int Lk, int ds, int wl,
                                                  int wr, int& lo, int& hi) {
  int l0, u0, l1, u1;
  key_steps_of(max(ia + Lk - Lq, 0), ds, Lk, l0, u0);
  key_steps_of(max(ib + Lk - Lq, 0), ds, Lk, l1, u1);
  lo = l0;
  hi = u1;
  if (wl >= 0 || wr >= 0) {
    const int klo = wl >= 0 ? max(0, ia + Lk - Lq - wl) : 0;
    const int khi = wr >= 0 ? min(Lk - 1, ib + Lk - Lq + wr) : Lk - 1;
    if (klo > khi) {
      lo = 0x7fffffff;
      hi = 0;
      return;
    }
    lo = max(lo, klo / TILE_ROWS);
    hi = min(hi, khi / TILE_ROWS + 1);
    if (lo >= hi) {
      lo = 0x7fffffff;
      hi = 0;
    }
  }
}

__device__ __forceinline__ void row_key_steps(bool exists, float slope2, int centre, int Lk,
                                              float thr, int& lo, int& hi) {
  lo = 0x7fffffff;
  hi = 0;
  if (!exists) return;
  key_steps_of(centre, key_half_width(slope2, Lk, thr), Lk, lo, hi);
}

// Offset of plan sequence v's first slope: packed sequence v / hkv, query
// heads from (v % hkv) * group (the slopes are [batch, hq], row stride given).
__device__ __forceinline__ int64_t slope_base(int v, int hkv, int group, int64_t stride) {
  const int b = v / hkv;
  return (int64_t)b * stride + (int64_t)(v - b * hkv) * group;
}

// Limits of the forward's longest-first list (each workgroup ranks every tile
// in LDS, fwd_impl.hpp): plan sequences, (plan sequence, head) pairs, row
// tiles, and rounds of the snake a workgroup resolves in advance.
constexpr int LPT_MAX_SEQS = 64;
constexpr int LPT_MAX_HEADS = 4096;
constexpr int LPT_MAX_TILES = 2048;
constexpr int FWD_LIST_MAX = 16;

// Planner (one workgroup), for the calls whose forward grid does not hold it.
hipError_t launch_prep(const PlanArgs& pa, hipStream_t s);
// Forward over the a.fwd_slots row-tile slots, with the planner (pa) in an
// extra workgroup beside them; with_delta (the full-VJP call) also plans the
// dK/dV units there and writes the row records.  One instantiation per head
// dimension D (fwd_d<D>.hip and so on); the dispatchers below pick it.
template <int D>
hipError_t launch_fwd_d(const AttnArgs& a, const PlanArgs& pa, int dtype, bool cap,
                        bool with_delta, hipStream_t s);
template <int D>
hipError_t launch_dkdv_d(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s);
template <int D>
hipError_t launch_dq_d(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s);
extern template hipError_t launch_fwd_d<64>(const AttnArgs&, const PlanArgs&, int, bool, bool,
                                            hipStream_t);
extern template hipError_t launch_fwd_d<128>(const AttnArgs&, const PlanArgs&, int, bool, bool,
                                             hipStream_t);
extern template hipError_t launch_fwd_d<160>(const AttnArgs&, const PlanArgs&, int, bool, bool,
                                             hipStream_t);
extern template hipError_t launch_dkdv_d<64>(const AttnArgs&, int, bool, int, hipStream_t);
extern template hipError_t launch_dkdv_d<128>(const AttnArgs&, int, bool, int, hipStream_t);
extern template hipError_t launch_dkdv_d<160>(const AttnArgs&, int, bool, int, hipStream_t);
extern template hipError_t launch_dq_d<64>(const AttnArgs&, int, bool, int, hipStream_t);
extern template hipError_t launch_dq_d<128>(const AttnArgs&, int, bool, int, hipStream_t);
extern template hipError_t launch_dq_d<160>(const AttnArgs&, int, bool, int, hipStream_t);

inline hipError_t launch_fwd(const AttnArgs& a, const PlanArgs& pa, int dtype, int d, bool cap,
                             bool with_delta, hipStream_t s) {
  switch (d) {
    case 64: return launch_fwd_d<64>(a, pa, dtype, cap, with_delta, s);
    case 128: return launch_fwd_d<128>(a, pa, dtype, cap, with_delta, s);
    default: return launch_fwd_d<160>(a, pa, dtype, cap, with_delta, s);
  }
}
inline hipError_t launch_dkdv(const AttnArgs& a, int dtype, int d, bool cap, int grid,
                              hipStream_t s) {
  switch (d) {
    case 64: return launch_dkdv_d<64>(a, dtype, cap, grid, s);
    case 128: return launch_dkdv_d<128>(a, dtype, cap, grid, s);
    default: return launch_dkdv_d<160>(a, dtype, cap, grid, s);
  }
}
inline hipError_t launch_dq(const AttnArgs& a, int dtype, int d, bool cap, int grid,
                            hipStream_t s) {
  switch (d) {
    case 64: return launch_dq_d<64>(a, dtype, cap, grid, s);
    case 128: return launch_dq_d<128>(a, dtype, cap, grid, s);
    default: return launch_dq_d<160>(a, dtype, cap, grid, s);
  }
}
hipError_t launch_rowinfo(const AttnArgs& a, int dtype, int d, bool cap, hipStream_t s);
// Sets *ticket = 0 on the stream (a one-thread launch, safe to capture).
hipError_t launch_ticket_reset(int* ticket, hipStream_t s);
// Key-step ranges of the standalone backward, from the row records, and its
// dK/dV units planned from them.
hipError_t launch_ksteps(const AttnArgs& a, int grid, hipStream_t s);
hipError_t launch_units(const PlanArgs& pa, hipStream_t s);

}  // namespace rga
