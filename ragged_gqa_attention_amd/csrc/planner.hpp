// Planning helpers shared by the prep kernel (plan.hip) and the forward
// kernel, whose extra workgroup plans the dK/dV units while the row tiles run.
#pragma once

#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

// Extents of plan sequence v (packed sequence v / hkv) from cu_q / cu_k, and
// whether they fail the planner's checks (see plan_block).
struct SeqExt {
  int cq, nq, ck, nk;
  bool bad;
};
__device__ __forceinline__ SeqExt seq_extents(const PlanArgs& pa, int v) {
  const int b = v / pa.hkv, nb = pa.batch / pa.hkv;
  SeqExt e;
  e.cq = pa.cu_q[b];
  e.nq = pa.cu_q[b + 1];
  e.ck = pa.cu_k[b];
  e.nk = pa.cu_k[b + 1];
  e.bad = e.cq < 0 || e.nq < e.cq || (int64_t)e.nq > pa.total_q || e.ck < 0 || e.nk < e.ck ||
          (int64_t)e.nk > pa.total_k;
  if (b == 0) e.bad |= e.cq != 0 || e.ck != 0;
  if (b == nb - 1) e.bad |= (int64_t)e.nq != pa.total_q || (int64_t)e.nk != pa.total_k;
  return e;
}

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
__device__ __forceinline__ void tile_key_steps(const int* s, int t, const int* hw, int wl, int wr,
                                               int& lo, int& hi) {
  const int Lq = s[SQ_LQ], Lk = s[SQ_LK], rows = s[SQ_ROWS];
  const int R0 = t * ROW_TILE, R1 = min(rows, R0 + ROW_TILE);
  const int hfirst = R0 / Lq, hlast = (R1 - 1) / Lq;
  lo = 0x7fffffff;
  hi = 0;
  for (int h = hfirst; h <= hlast; ++h) {
    const int ia = h == hfirst ? R0 - h * Lq : 0;
    const int ib = h == hlast ? R1 - 1 - h * Lq : Lq - 1;
    int l, u;
    token_range_steps(ia, ib, Lq, Lk, hw[h], wl, wr, l, u);
    if (l < u) {
      lo = min(lo, l);
      hi = max(hi, u);
    }
  }
  finish_range(lo, hi);
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

// Batches up to this size are planned in LDS and copied out at the end (each
// planning step re-reads what the previous one wrote; LDS keeps those round
// trips short); larger ones are planned in place in global memory.
constexpr int PLAN_LDS_B = 256;
// Row tiles are dispatched longest first (by their key steps, counting-sorted
// into this many classes; longer ones share the last class).  Tiles of equal
// length go in the order the LDS atomics hand out, which only affects timing:
// a tile's results do not depend on the workgroup that computes it.
constexpr int PLAN_COST_CLASSES = 1024;
// Row tiles whose sequence the planner looks up in an LDS table (the rest by
// binary search).
constexpr int PLAN_LDS_TILES = 4096;

// LDS of plan_block (up to 16 waves).
struct PlanShared {
  long long red[16];
  int part[16];
  int seq[PLAN_LDS_B * SEQ_FIELDS];
  int hw[PLAN_LDS_HEADS];
  int cls[PLAN_COST_CLASSES + 1];
  int foff[PLAN_COST_CLASSES];
  int tseq[PLAN_LDS_TILES];
};

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
    e[KV_HB] = s[SQ_HB]; e[KV_G] = s[SQ_G]; e[KV_PAD0] = 0;
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

template <int NT>
__device__ __forceinline__ void plan_block(const PlanArgs& a, PlanShared& sh) {
  long long* red = sh.red;
  int* part = sh.part;
  int* l_seq = sh.seq;
  int* l_hw = sh.hw;
  int* l_class = sh.cls;
  int* l_foff_c = sh.foff;
  int* l_tseq = sh.tseq;
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int hq = a.hq;
  const bool in_lds = B <= PLAN_LDS_B;
  int* seq = in_lds ? l_seq : a.plan.seq;

  if (tid < 32) reinterpret_cast<u32x4*>(a.zero)[tid] = u32x4{0u, 0u, 0u, 0u};
  // the slopes, requested first (their loads overlap those of the checks
  // below); thread tid takes (sequence, head) pairs tid + 256 k
  constexpr int SPER = PLAN_LDS_HEADS / NT;
  const bool hw_lds = (long long)B * hq <= PLAN_LDS_HEADS;
  const int sb0 = tid / hq, sh0 = tid - sb0 * hq;   // pair tid
  const int sdb = NT / hq, sdh = NT - sdb * hq;
  float sv[SPER];
  if (hw_lds && B > 0) {   // unconditional loads (pairs past the last read (B - 1, h)), all in flight at once
    int b = sb0, h = sh0;
#pragma unroll
    for (int k = 0; k < SPER; ++k) {
      sv[k] = a.slopes[slope_base(min(b, B - 1), a.hkv, hq, a.slopes_stride) + h];
      b += sdb;
      h += sdh;
      if (h >= hq) { h -= hq; ++b; }
    }
  }
  // checks of cu_q / cu_k and the per-sequence extents in one pass (plan
  // sequence v = packed sequence v / hkv, K/V head v % hkv); an invalid batch
  // is then planned with every sequence empty
  auto extents = [&](int v, int q0, int lq, int k0, int lk) {
    int* s = seq + v * SEQ_FIELDS;
    s[SQ_Q0] = q0; s[SQ_LQ] = lq; s[SQ_K0] = k0; s[SQ_LK] = lk;
    s[SQ_ROWS] = lq * a.hq;
    s[SQ_KTILES] = (lk + KEY_TILE - 1) / KEY_TILE;
    uint32_t mul, sh;
    fast_div_consts(lq, mul, sh);
    s[SQ_LQSHIFT] = (int)sh;
    s[SQ_LQMUL] = (int)mul;
    const int g = v - (v / a.hkv) * a.hkv;
    s[SQ_HB] = g * a.hq;
    s[SQ_G] = g;
  };
  // an empty batch still has cu[0], which must be 0 = total
  bool bad = B == 0 && tid == 0 &&
             (a.cu_q[0] != 0 || a.cu_k[0] != 0 || a.total_q != 0 || a.total_k != 0);
  for (int v = tid; v < B; v += NT) {
    const SeqExt e = seq_extents(a, v);
    bad |= e.bad;
    // (a failed check leaves this sequence empty, so no length is negative)
    if (e.bad) extents(v, 0, 0, 0, 0);
    else extents(v, e.cq, e.nq - e.cq, e.ck, e.nk - e.ck);
  }
  const bool ok = __syncthreads_or(bad) == 0;
  if (tid == 0) a.plan.flag[0] = ok ? 0 : 1;
  if (!ok) {
    for (int b = tid; b < B; b += NT) extents(b, 0, 0, 0, 0);
    __syncthreads();
  }

  // 256-row tiles in batch order (their key-step ranges are kept in this
  // order); tile -> sequence in LDS when the tiles fit
  block_exclusive_scan<NT>(B, [&](int b) {
    return (seq[b * SEQ_FIELDS + SQ_ROWS] + ROW_TILE - 1) / ROW_TILE;
  }, [&](int b, int v) {
    if (b >= B) return;
    seq[b * SEQ_FIELDS + SQ_RTOFF] = v;
    const int n = (seq[b * SEQ_FIELDS + SQ_ROWS] + ROW_TILE - 1) / ROW_TILE;
    for (int t = v; t < min(v + n, PLAN_LDS_TILES); ++t) l_tseq[t] = b;
  }, part);
  const int nrt = B > 0 ? seq[(B - 1) * SEQ_FIELDS + SQ_RTOFF] +
                              (seq[(B - 1) * SEQ_FIELDS + SQ_ROWS] + ROW_TILE - 1) / ROW_TILE
                        : 0;

  // Key-step range of every row tile (see tile_key_steps), from each head's
  // key half-width (LDS, from the slopes requested at the start, when they
  // fit; else the workspace, eight slope loads in flight per thread).
  int* hw = hw_lds ? l_hw : a.head_hw;
  if (hw_lds) {
    int b = sb0, h = sh0;
#pragma unroll
    for (int k = 0; k < SPER; ++k) {
      if (b < B)
        hw[b * hq + h] = key_half_width(sv[k] * LOG2E, seq[b * SEQ_FIELDS + SQ_LK], a.skip_log2);
      b += sdb;
      h += sdh;
      if (h >= hq) { h -= hq; ++b; }
    }
  } else {
    constexpr int PER = 8;
    for (int i0 = 0; i0 < B * hq; i0 += NT * PER) {
      float v[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = i0 + k * NT + tid;
        const int b = i / hq;
        v[k] = i < B * hq ? a.slopes[slope_base(b, a.hkv, hq, a.slopes_stride) + (i - b * hq)]
                          : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = i0 + k * NT + tid;
        if (i < B * hq)
          hw[i] = key_half_width(v[k] * LOG2E, seq[(i / hq) * SEQ_FIELDS + SQ_LK], a.skip_log2);
      }
    }
  }
  for (int i = tid; i <= PLAN_COST_CLASSES; i += NT) l_class[i] = 0;
  __threadfence_block();
  __syncthreads();
  auto seq_of_tile = [&](int g) {
    if (g < PLAN_LDS_TILES) return l_tseq[g];
    return last_at_most(B, g, [&](int x) { return seq[x * SEQ_FIELDS + SQ_RTOFF]; });
  };
  for (int g = tid; g < nrt; g += NT) {
    const int b = seq_of_tile(g);
    const int* s = seq + b * SEQ_FIELDS;
    int lo, hi;
    tile_key_steps(s, g - s[SQ_RTOFF], hw + b * hq, a.win_left, a.win_right, lo, hi);
    a.ksteps[2 * g] = lo;
    a.ksteps[2 * g + 1] = hi;
    // class 0 holds the longest tiles
    atomicAdd(&l_class[PLAN_COST_CLASSES - 1 - min(max(hi - lo, 0), PLAN_COST_CLASSES - 1)], 1);
  }
  __syncthreads();
  // workgroup -> row tile, longest first; entries past the last tile get
  // sequence -1
  block_exclusive_scan<NT>(PLAN_COST_CLASSES, [&](int c) { return l_class[c]; },
                                     [&](int c, int v) { if (c < PLAN_COST_CLASSES) l_foff_c[c] = v; },
                                     part);
  for (int g = tid; g < nrt; g += NT) {
    const int lo = a.ksteps[2 * g], hi = a.ksteps[2 * g + 1];
    const int pos =
        atomicAdd(&l_foff_c[PLAN_COST_CLASSES - 1 - min(max(hi - lo, 0), PLAN_COST_CLASSES - 1)], 1);
    const int b = seq_of_tile(g);
    a.plan.fwd_map[2 * pos] = b;
    a.plan.fwd_map[2 * pos + 1] = g - seq[b * SEQ_FIELDS + SQ_RTOFF];
  }
  for (int i = nrt + tid; i < a.fwd_slots; i += NT) {
    a.plan.fwd_map[2 * i] = -1;
    a.plan.fwd_map[2 * i + 1] = 0;
  }
  if (tid == 0) a.plan.kv_head[2] = nrt;
  // 128-key tiles in batch order (dK / dV units and partial sums walk them)
  block_exclusive_scan<NT>(B, [&](int b) { return seq[b * SEQ_FIELDS + SQ_KTILES]; },
                       [&](int b, int v) { if (b < B) seq[b * SEQ_FIELDS + SQ_KTOFF] = v; }, part);
  // stored dS images, in sequence order, while they fit the workspace (a
  // sequence that does not fit recomputes dS in the dQ kernel)
  auto images = [&](int b) -> long long {
    const int* sb = seq + b * SEQ_FIELDS;
    if (sb[SQ_ROWS] == 0 || sb[SQ_LK] == 0) return 0;
    return (long long)((sb[SQ_ROWS] + ROW_TILE - 1) / ROW_TILE) *
           ((sb[SQ_LK] + TILE_ROWS - 1) / TILE_ROWS);
  };
  block_exclusive_scan<NT>(B, images, [&](int b, long long off) {
    if (b < B) {
      const long long n = images(b);
      seq[b * SEQ_FIELDS + SQ_DSOFF] = (n > 0 && off + n <= a.ds_images) ? (int)off : -1;
    }
  }, red);

  if (in_lds) {   // the kernels read the plan from global memory
    for (int i = tid; i < B * SEQ_FIELDS; i += NT) a.plan.seq[i] = l_seq[i];
  }
}

// ---------------------------------------------------------------------------
// A forward workgroup's row tile, found without the planner so the forward
// need not wait for it.  The 256-row tiles of the batch are taken in an order
// computable from cu_q / cu_k alone: sequences by key length, longest first
// (ties by index), when there are at most 64 of them, else in batch order;
// slot i gets tile i of that order (long tiles start first, short ones fill
// the tail).  Every wave computes the same answer from the same loads (no
// LDS, no barrier).  cu_q / cu_k are checked as the planner checks them.
struct RowTile {
  int b, tile;          // sequence, 256-row tile of the sequence
  int q0, lq, k0, lk;   // the sequence's extents
};

// false past the last tile, or when cu_q / cu_k are invalid (the planner
// flags that case and plans nothing).  b is a plan sequence (see SeqField).
__device__ __forceinline__ bool find_row_tile(const PlanArgs& pa, int slot, RowTile& t) {
  const int lane = threadIdx.x & 63;
  const int B = pa.batch, hq = pa.hq;
  if (B <= 0) return false;
  if (B <= 64) {
    const int b = lane;
    const bool live = b < B;
    // unconditional loads (lanes past B - 1 repeat the last sequence), so
    // the four requests are in flight together
    SeqExt e = seq_extents(pa, min(b, B - 1));
    if (!live) e.cq = e.nq = e.ck = e.nk = 0;
    if (__any(live && e.bad)) return false;
    const int lq = e.nq - e.cq, lk = e.nk - e.ck;
    const int n = live ? (lq * hq + ROW_TILE - 1) / ROW_TILE : 0;
    // first tile of sequence b: the tiles of the sequences ranked before it
    int start = 0;
    for (int j = 0; j < B; ++j) {
      const int lkj = __builtin_amdgcn_readlane(lk, j), nj = __builtin_amdgcn_readlane(n, j);
      start += (lkj > lk || (lkj == lk && j < b)) ? nj : 0;
    }
    const uint64_t own = __ballot(live && start <= slot && slot < start + n);
    if (own == 0) return false;
    const int ob = __ffsll((long long)own) - 1;
    t.b = ob;
    t.tile = slot - __builtin_amdgcn_readlane(start, ob);
    t.q0 = __builtin_amdgcn_readlane(e.cq, ob);
    t.lq = __builtin_amdgcn_readlane(lq, ob);
    t.k0 = __builtin_amdgcn_readlane(e.ck, ob);
    t.lk = __builtin_amdgcn_readlane(lk, ob);
    return true;
  }
  // batch order: lane l owns plan sequences [l seg, l seg + seg)
  const int seg = (B + 63) / 64;
  const int lo = min(B, lane * seg), hi = min(B, lo + seg);
  bool bad = false;
  int count = 0;
  for (int b = lo; b < hi; ++b) {
    const SeqExt e = seq_extents(pa, b);
    bad |= e.bad;
    count += ((e.nq - e.cq) * hq + ROW_TILE - 1) / ROW_TILE;
  }
  if (__any(bad)) return false;
  int x = count;   // inclusive scan over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  const int run0 = x - count;
  const uint64_t own = __ballot(run0 <= slot && slot < x);
  if (own == 0) return false;
  const int ol = __ffsll((long long)own) - 1;
  if (lane == ol) {
    int run = run0;
    for (int b = lo; b < hi; ++b) {
      const SeqExt e = seq_extents(pa, b);
      const int n = ((e.nq - e.cq) * hq + ROW_TILE - 1) / ROW_TILE;
      if (slot < run + n) {
        t.b = b;
        t.tile = slot - run;
        t.q0 = e.cq;
        t.lq = e.nq - e.cq;
        t.k0 = e.ck;
        t.lk = e.nk - e.ck;
        break;
      }
      run += n;
    }
  }
  t.b = __builtin_amdgcn_readlane(t.b, ol);
  t.tile = __builtin_amdgcn_readlane(t.tile, ol);
  t.q0 = __builtin_amdgcn_readlane(t.q0, ol);
  t.lq = __builtin_amdgcn_readlane(t.lq, ol);
  t.k0 = __builtin_amdgcn_readlane(t.k0, ol);
  t.lk = __builtin_amdgcn_readlane(t.lk, ol);
  return true;
}

// The tile's key-step range, equal to the planner's tile_key_steps: each head
// the tile spans (one per lane, 64 at a time) contributes the ranges of its
// first and its last row of the tile, from its half-width key_half_width.
__device__ __forceinline__ void tile_key_range(const PlanArgs& pa, const RowTile& t, int& lo,
                                               int& hi) {
  const int lane = threadIdx.x & 63;
  const int rows = t.lq * pa.hq;
  const int R0 = t.tile * ROW_TILE, R1 = min(rows, R0 + ROW_TILE);
  const int hfirst = R0 / t.lq, hlast = (R1 - 1) / t.lq;
  lo = 0x7fffffff;
  hi = 0;
  for (int h0 = hfirst; h0 <= hlast; h0 += 64) {
    const int h = h0 + lane;
    if (h <= hlast) {
      const float slope = pa.slopes[slope_base(t.b, pa.hkv, pa.hq, pa.slopes_stride) + h];
      const int hw = key_half_width(slope * LOG2E, t.lk, pa.skip_log2);
      const int ia = h == hfirst ? R0 - h * t.lq : 0;
      const int ib = h == hlast ? R1 - 1 - h * t.lq : t.lq - 1;
      int l, u;
      token_range_steps(ia, ib, t.lq, t.lk, hw, pa.win_left, pa.win_right, l, u);
      if (l < u) {
        lo = min(lo, l);
        hi = max(hi, u);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  finish_range(lo, hi);
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
}


}  // namespace rga
