// Planning helpers shared by the prep kernel (plan.hip) and the forward
// kernel, whose extra workgroup plans the dK/dV units while the row tiles run.
#pragma once

#include "kernels.hpp"

namespace rga {

// Block-wide helpers of the planners, for workgroups of NT threads (NT / 64
// waves); `red` / `part` are LDS arrays of one entry per wave.

// Sum over the block (wave shuffles, then the wave totals).
template <int NT>
__device__ __forceinline__ long long block_sum(long long v, long long* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  long long r = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

// put(r, sum_{r' < r} count(r')) for r = 0..B.  Thread t owns a contiguous
// segment of r; segment totals are scanned with wave shuffles.
template <int NT, class V, class F, class G>
__device__ __forceinline__ void block_exclusive_scan(int B, F count, G put, V* part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (B + NT - 1) / NT;
  const int lo = min(B, tid * seg), hi = min(B, lo + seg);
  V local = 0;
  for (int r = lo; r < hi; ++r) local += count(r);
  V x = local;   // inclusive scan inside the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  V base = 0;
  for (int w = 0; w < wave; ++w) base += part[w];
  if (tid == NT - 1) put(B, base + x);
  V run = base + x - local;
  for (int r = lo; r < hi; ++r) {
    put(r, run);
    run += count(r);
  }
  __syncthreads();
}

// Batches with up to this many 128-key tiles count each key tile's visited
// row tiles exactly (in LDS); larger ones plan as if every row tile visited
// every key tile (the dK/dV kernel still skips, units just come out uneven).
constexpr int PLAN_LDS_KT = 2048;

// Key-step range [lo, hi) of row tile t of a sequence (record s; the
// half-widths key_half_width of its heads at hw[h]): min / max of
// row_key_steps over its rows.  For one head both bounds grow with the token
// (the centre does), so each head the tile spans contributes its first and
// its last row.
__device__ __forceinline__ void tile_key_steps(const int* s, int t, const int* hw, int& lo,
                                               int& hi) {
  const int Lq = s[SQ_LQ], Lk = s[SQ_LK], rows = s[SQ_ROWS];
  const int R0 = t * ROW_TILE, R1 = min(rows, R0 + ROW_TILE);
  const int hfirst = R0 / Lq, hlast = (R1 - 1) / Lq;
  lo = 0x7fffffff;
  hi = 0;
  for (int h = hfirst; h <= hlast; ++h) {
    const int ia = h == hfirst ? R0 - h * Lq : 0;
    const int ib = h == hlast ? R1 - 1 - h * Lq : Lq - 1;
    int l0, u0, l1, u1;
    key_steps_of(max(ia + Lk - Lq, 0), hw[h], Lk, l0, u0);
    key_steps_of(max(ib + Lk - Lq, 0), hw[h], Lk, l1, u1);
    lo = min(lo, l0);
    hi = max(hi, u1);
  }
}

// Last index r in [0, n) with key(r) <= x (key nondecreasing, key(0) <= x).
template <class F>
__device__ __forceinline__ int last_at_most(int n, int x, F key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Per-head key half-widths the prep planner keeps in LDS while it evaluates
// tile ranges (batches with more (sequence, head) pairs keep them in the
// workspace).
constexpr int PLAN_LDS_HEADS = 4096;

// dK/dV work split, planned by one workgroup of NT threads from the row
// tiles' key-step ranges in a.ksteps (seq: the sequence records).
//
// A 128-key tile is visited by the row tiles whose range meets its two key
// steps; V counts their 64-row steps (a difference array over the sequence's
// key tiles and a prefix sum).  The key tiles, in batch order, form one list
// of W items: key tile g holds a_seg leading items that stand for the fixed
// cost of starting a segment (loading K / V, the pipeline's first and last
// steps), then its V visit steps, items [S_g, S_g + a_seg + V_g) (nothing when
// V_g = 0).  dK/dV workgroup p of kv_wgs takes items [p W / kv_wgs,
// (p + 1) W / kv_wgs), so the workgroups get near-equal modelled work.  Key
// tiles whose visit steps fall to several workgroups are summed from FP32
// partials afterwards.  The planner writes one record per key tile (KvField;
// a workgroup reads a record with one load), the first key tile of every
// workgroup, and W, the key tile count and a_seg in kv_head.
struct UnitsShared {
  long long red[16];   // one slot per wave
  int part[16];
  int total;
  int kvis[PLAN_LDS_KT], kex[PLAN_LDS_KT + 1];
};

template <int NT>
__device__ __forceinline__ void plan_units(const PlanArgs& a, const int* seq, UnitsShared& sh) {
  static_assert(NT / 64 <= 16, "per-wave LDS slots");
  int* part = sh.part;
  int* l_kvis = sh.kvis;
  int* l_kex = sh.kex;
  const int tid = threadIdx.x;
  const int B = a.batch;
  int nrt = 0, nkt = 0;
  if (B > 0) {
    const int* s = seq + (B - 1) * SEQ_FIELDS;
    nrt = s[SQ_RTOFF] + (s[SQ_ROWS] + ROW_TILE - 1) / ROW_TILE;
    nkt = s[SQ_KTOFF] + s[SQ_KTILES];
  }
  const bool exact = nkt <= PLAN_LDS_KT;
  auto seq_of_tile = [&](int g) {
    return last_at_most(B, g, [&](int x) { return seq[x * SEQ_FIELDS + SQ_RTOFF]; });
  };
  auto seq_of_ktile = [&](int g) {
    return last_at_most(B, g, [&](int x) { return seq[x * SEQ_FIELDS + SQ_KTOFF]; });
  };
  for (int i = tid; i < PLAN_LDS_KT; i += NT) l_kvis[i] = 0;
  __syncthreads();
  for (int g = tid; g < nrt; g += NT) {
    const int b = seq_of_tile(g);
    const int* s = seq + b * SEQ_FIELDS;
    const int lo = a.ksteps[2 * g], hi = a.ksteps[2 * g + 1];
    if (exact && hi > lo) {
      const int kt_lo = lo / 2, kt_hi = (hi - 1) / 2;   // key tiles of 2 key steps
      // 64-row steps of the tile (only a sequence's last tile has fewer than 4)
      const int rest = s[SQ_ROWS] - (g - s[SQ_RTOFF]) * ROW_TILE;
      const int steps = min(ROW_TILE / KV_ROW_STEP, (rest + KV_ROW_STEP - 1) / KV_ROW_STEP);
      atomicAdd(&l_kvis[s[SQ_KTOFF] + kt_lo], steps);
      if (kt_hi + 1 < s[SQ_KTILES]) atomicAdd(&l_kvis[s[SQ_KTOFF] + kt_hi + 1], -steps);
    }
  }
  __syncthreads();
  if (exact) {
    block_exclusive_scan<NT>(nkt, [&](int g) { return l_kvis[g]; },
                             [&](int g, int v) { l_kex[g] = v; }, part);
    for (int g = tid; g < nkt; g += NT) {
      const int b = seq_of_ktile(g);
      l_kvis[g] = l_kex[g] + l_kvis[g] - l_kex[seq[b * SEQ_FIELDS + SQ_KTOFF]];
    }
    __syncthreads();
  }
  auto visits = [&](int g) {
    if (exact) return l_kvis[g];
    const int* s = seq + seq_of_ktile(g) * SEQ_FIELDS;
    return (s[SQ_ROWS] + KV_ROW_STEP - 1) / KV_ROW_STEP;
  };
  auto items = [&](int g) { const int v = visits(g); return v > 0 ? v + a.seg_items : 0; };
  // key tile records; item starts S_g (kept in LDS when they fit)
  block_exclusive_scan<NT>(nkt, items, [&](int g, int s0) {
    if (g == nkt) {
      sh.total = s0;
      return;
    }
    if (exact) l_kex[g] = s0;
    const int b = seq_of_ktile(g);
    const int* s = seq + b * SEQ_FIELDS;
    int* e = a.plan.ktab + KV_FIELDS * g;
    e[KV_B] = b; e[KV_KTILE] = g - s[SQ_KTOFF]; e[KV_V] = visits(g); e[KV_S] = s0;
    e[KV_Q0] = s[SQ_Q0]; e[KV_K0] = s[SQ_K0]; e[KV_LK] = s[SQ_LK]; e[KV_ROWS] = s[SQ_ROWS];
    e[KV_RTOFF] = s[SQ_RTOFF]; e[KV_DSOFF] = s[SQ_DSOFF]; e[KV_LQ] = s[SQ_LQ];
    e[KV_LQMUL] = s[SQ_LQMUL]; e[KV_LQSHIFT] = s[SQ_LQSHIFT];
    e[KV_PAD0] = 0; e[KV_PAD1] = 0; e[KV_PAD2] = 0;
  }, part);
  __threadfence_block();
  __syncthreads();
  const long long W = sh.total;
  if (tid == 0) {
    a.plan.kv_head[0] = (int)W;
    a.plan.kv_head[1] = nkt;
    a.plan.kv_head[3] = a.seg_items;
  }
  // first key tile of every workgroup's share (-1 for an empty share)
  for (int p = tid; p < a.kv_wgs; p += NT) {
    const long long w0 = (long long)p * W / a.kv_wgs, w1 = (long long)(p + 1) * W / a.kv_wgs;
    int g = -1;
    if (w0 < w1)
      g = last_at_most(nkt, (int)w0, [&](int x) {
        return exact ? l_kex[x] : a.plan.ktab[KV_FIELDS * x + KV_S];
      });
    a.plan.wg_first[p] = g;
  }
}

}  // namespace rga
