// dK / dV kernel: recompute P from the stored row record, then
//   dP = dO V^T,  dS = P * (dP - Delta) * (1 - tanh^2(s / c)),
//   dV = sum_rows P^T dO,  dK = sigma sum_rows dS^T Q,
// summed over every folded (head, token) row of the plan sequence, i.e. over
// all query heads that share the K/V head.  Templated on the head dimension D
// (64, 128, 160); one translation unit per D.
//
// Page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section "Hard
// Constraints": the K/V gradients reduce over every query head sharing the K/V
// head, and the cap sits between the scaled dot product and ALiBi, so its
// derivative multiplies dP - Delta.  Page "python-20261012-ragged-flash-
// attention-gradient-recompute", section "Root causes addressed": no
// probability matrix is stored; each tile is rebuilt from L.
//
// With r = 1 / (1 + e^{2s/c}), 1 - tanh^2(s/c) = 4 r (1 - r); the kernel forms
// r - r^2 and folds the factor 4 into the final sigma scale of dK.
//
// Work split.  Every (128-key tile, 64-row step of a visiting row tile) pair
// of the batch is an item of a list the planner builds (see plan_units); each
// of the kv_wgs workgroups takes an equal share of consecutive items and walks
// them key tile by key tile: a segment is 128 keys of one sequence against a
// run of the row steps that visit them.  Its eight waves form four pairs; a pair owns 32 keys and keeps
// their K and V rows in registers (MFMA operands, lane = key).  Rows are
// streamed 64 at a time through LDS.  In each step the two waves of a pair
// each form S, dP, P and dS for one half of the rows (32 rows x 32 keys), then
// trade halves through LDS: the first wave accumulates dV = P^T dO over all 64
// rows, the second dK = dS^T Q.  Each wave thus holds one accumulator and
// stays within 256 registers, so two waves share each SIMD; they take the
// independent products and pointwise work of a step in opposite orders, so
// one wave's VALU work overlaps the other's MFMAs.  The sum over rows happens
// in registers in a fixed order; a key tile whose items fall to several
// workgroups is written as FP32 partials (a workgroup's first and last key
// tile) that a separate pass adds in workgroup order.  No atomics anywhere.
//
// Pipeline.  Q and dO tiles are copied global -> LDS with direct loads (no
// staging registers) into blocked tiles, three buffers: step n is read by the
// S/dP products, step n - 1 by the dV/dK products and step n + 1 is in flight.
//
// Far rows.  A 256-row tile whose recorded key steps (a.ksteps, see
// row_key_steps) miss the workgroup's 128 keys has P == 0 exactly on all of
// them, so its row steps are passed over; the steps a workgroup does visit
// therefore cover every dS image the dQ kernel later reads.
#pragma once

#include "dropout.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

namespace kvd {

constexpr int KV_NBUF = 3;
constexpr int KV_WAVES = KV_THREADS / 64;
constexpr int PAIR_KEYS = KEY_TILE / (KV_WAVES / 2);  // keys of one wave pair
constexpr int KB = PAIR_KEYS / 32;                    // 32-key blocks per wave
static_assert(KV_WAVES == 8 && KB == 1, "eight waves: wave w copies tensor w / 4, row group w % 4");
static_assert(KV_ROW_STEP == TILE_ROWS, "a step is one row tile (see blk_off)");

template <int D, bool DROP>
struct KvShared {
  uint16_t qd[KV_NBUF][2][tile_elems<D>()];   // Q and dO rows of a step (blocked)
  f32x4 rinfo[KV_NBUF][KV_ROW_STEP];     // row records of a step
  u32x4 xch[2][KV_WAVES][KB * 2][64];     // [slot][writer wave][kb * 2 + s][lane]
  u32x4 drec[DROP ? KV_NBUF : 1][DROP ? KV_ROW_STEP : 1];   // dropout records of a step
};

// What a segment works on: visiting 64-row steps number first .. last - 1 (in
// row order) of the 128-key tile, against keys [key0, key0 + PAIR_KEYS) of the
// wave's pair.  Every visiting row tile has four steps except a sequence's
// last, which comes last.
struct KvUnit {
  int q0, k0, Lk, rows, key0;
  int hb, kvh;              // first query head of the group, K/V head
  int64_t rbase;            // first row record of the plan sequence (q0 hq + hb Lq)
  int lq, lqmul, lqshift;   // unfold_row constants of the sequence
  int first, last;
  int part;  // FP32 partial slot of the segment, -1 when it stores dK / dV directly
  int ds;    // first dS image of the sequence, -1 when dS is not stored
  int nks;   // 64-key steps of the sequence (images per row tile)
  const int* ksteps;   // key-step ranges of the sequence's row tiles
  int step_lo;         // the workgroup's key steps [step_lo, step_lo + 2)
};

// Row tiles the workgroup visits, as a 64-tile bit mask (kept in scalar
// registers, reloaded past its end).
struct TileMask {
  uint64_t bits;
  int base;    // tile of bit 0
  int last;    // last tile of the row range
};

__device__ __forceinline__ void tile_mask_load(TileMask& m, const KvUnit& u, int base, int lane) {
  asm volatile("" : "+v"(lane));   // (per call: no hoisted per-lane addresses)
  const int t = base + lane;
  bool on = false;
  if (t <= m.last) {
    const int* r = u.ksteps + 2 * t;
    on = r[0] < u.step_lo + 2 && r[1] > u.step_lo;
  }
  m.bits = __ballot(on);
  m.base = base;
}

// First visited tile >= t, or a tile past m.last.
__device__ __forceinline__ int tile_mask_next(TileMask& m, const KvUnit& u, int t, int lane) {
  while (t <= m.last) {
    if (t >= m.base + 64) tile_mask_load(m, u, t, lane);
    const uint64_t rest = m.bits >> (t - m.base);
    if (rest != 0) return t + (int)__builtin_ctzll(rest);
    t = m.base + 64;
  }
  return t;
}

// The work of one wave; ROLE 0 accumulates dV, ROLE 1 dK.
template <class T, int D, bool CAP, int ROLE, bool LATE, bool WIN, bool DROP>
__device__ __forceinline__ void dkdv_wave(const AttnArgs& a, KvShared<D, DROP>& sm,
                                          const KvUnit& u, int wave, int lane) {
  constexpr int KSTEPS = Geo<D>::KSTEPS, DBLK = Geo<D>::DBLK, CHUNKS = Geo<D>::CHUNKS;
  constexpr int LOADS_PER_WAVE = CHUNKS / 4;   // 4-chunk blocks of a 16-row group
  const int l32 = lane & 31, g = lane >> 5;

  // whether row tile t visits the key tile (its key-step range meets the
  // key tile's two steps); the first 64 are requested before the K / V rows
  const int ntile = (u.rows + ROW_TILE - 1) / ROW_TILE;
  auto visits = [&](int t) {
    if (t >= ntile) return false;
    const int* r = u.ksteps + 2 * t;
    return r[0] < u.step_lo + 2 && r[1] > u.step_lo;
  };
  const bool on0 = visits(lane);

  // K and V rows of the pair's keys as B operands (lane = key); keys past
  // the sequence end are zero and their results are never stored.
  u32x4 kf[KB][KSTEPS], vf[KB][KSTEPS];
  float keyf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = u.key0 + kb * 32 + l32;
    keyf[kb] = (float)key;
    const bool ok = key < u.Lk;
    const uint16_t* kr =
        a.k + (int64_t)(u.k0 + (ok ? key : 0)) * a.k_ts + (int64_t)u.kvh * a.k_hs + g * 8;
    const uint16_t* vr =
        a.v + (int64_t)(u.k0 + (ok ? key : 0)) * a.v_ts + (int64_t)u.kvh * a.v_hs + g * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 kx = load16(kr + ks * 16), vx = load16(vr + ks * 16);
      kf[kb][ks] = ok ? kx : u32x4{0u, 0u, 0u, 0u};
      vf[kb][ks] = ok ? vx : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // The segment's run: its first and last steps lie in the visiting tiles of
  // ranks first / 4 and (last - 1) / 4, found in one pass over the row
  // tiles, 64 per ballot (lane l examines tile base + l), while the K / V
  // loads are in flight; the window holding the first tile seeds the tile
  // mask.  rb, re: rows [rb, re) from the first to the end of the last step.
  // The first step's copies are requested as soon as rb is known.
  int rb = 0, re = 0;
  TileMask tm;
  tm.bits = 0;
  tm.base = 0;
  tm.last = -1;
  {
    constexpr int TS = ROW_TILE / KV_ROW_STEP;   // steps per row tile
    const int first = u.first / TS, last = (u.last - 1) / TS + 1;   // tile ranks
    const uint64_t below = (1ull << lane) - 1;   // lanes under this one
    int seen = 0, t_first = -1, t_last = -1;
    for (int base = 0; first < last && base < ntile && t_last < 0; base += 64) {
      const bool on = base == 0 ? on0 : visits(base + lane);
      const uint64_t m = __ballot(on);
      const int rank = seen + __popcll(m & below);   // visited tiles before this lane's
      const int c = __popcll(m);
      if (t_first < 0 && seen + c > first) {
        t_first = base + __builtin_ctzll(__ballot(on && rank == first));
        tm.bits = m;
        tm.base = base;
      }
      if (seen + c >= last) t_last = base + __builtin_ctzll(__ballot(on && rank == last - 1));
      seen += c;
    }
    if (t_first >= 0 && t_last >= t_first) {
      rb = t_first * ROW_TILE + (u.first % TS) * KV_ROW_STEP;
      re = min(u.rows, t_last * ROW_TILE + ((u.last - 1) % TS + 1) * KV_ROW_STEP);
      tm.last = t_last;
    }
  }

  // Direct loads of step rows [r0, r0 + 64) into blocked tiles (see blk_off):
  // wave w copies rows 16 (w%4) .. +15 of Q (w < 4) or dO, one 4-chunk block
  // per load, lane l holding row 16 (w%4) + l / 4 for all five loads, so one
  // address per lane per step.  Rows past the chunk end read the zero block.  Wave 0
  // also copies the 64 row records.
  const int lgroup = wave & 3;            // 16-row group this wave copies
  const int ltensor = wave >> 2;          // 0: Q, 1: dO
  auto issue_loads = [&](int r0, int buf) {
    // the lane's row and chunk are recomputed per step (an empty asm keeps
    // the compiler from hoisting them into registers it would then spill)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lrow = 16 * lgroup + (ln >> 2);
    const int lchunk = (ln & 3) ^ ((ln >> 4) & 3);
    if (wave == 0) {
      const int R = r0 + lane;
      const float* src = a.rowinfo + (u.rbase + min(R, re - 1)) * 4;
      load_lds16_unseen(R < re ? (const void*)src : (const void*)a.zero, &sm.rinfo[buf][0]);
    }
    if (DROP && wave == 1) {
      const int R = r0 + lane;
      const u32x4* src = a.droprec + u.rbase + min(R, re - 1);
      load_lds16_unseen(R < re ? (const void*)src : (const void*)a.zero, &sm.drec[buf][0]);
    }
    const int R = r0 + lrow;
    const int Rc = min(R, re - 1);
    int tok_, h_;
    // (uniform: kept in scalar registers rather than spilled vector ones)
    unfold_row(Rc, __builtin_amdgcn_readfirstlane(u.lq),
               (uint32_t)__builtin_amdgcn_readfirstlane(u.lqmul),
               (uint32_t)__builtin_amdgcn_readfirstlane(u.lqshift), tok_, h_);
    const uint32_t tok = (uint32_t)tok_, h = (uint32_t)(h_ + u.hb);
    const uint32_t t_abs = (uint32_t)u.q0 + tok;
    const bool ok = R < re;
    const uint16_t* base = ltensor ? a.dout : a.q;
    const uint32_t ts = (uint32_t)(ltensor ? a.do_ts : a.q_ts);
    const uint32_t hs = (uint32_t)(ltensor ? a.do_hs : a.q_hs);
    const uint16_t* src = (ok ? base + ((uint64_t)t_abs * ts + (uint64_t)h * hs) : a.zero) + lchunk * 8;
#pragma unroll
    for (int p = 0; p < LOADS_PER_WAVE; ++p)
      load_lds16_unseen(src + p * 32, &sm.qd[buf][ltensor][(lgroup * LOADS_PER_WAVE + p) * BLK_ELEMS]);
  };

  // Lane-constant LDS offsets (elements).  Row reads of the S / dP A operand:
  // row ROLE * 32 + l32, chunk 2 ks + g; ks / 2 selects the block column and
  // ks % 2 the XOR pattern.
  const int arow = ROLE * 32 + l32;
  const int roff[2] = {blk_off<D>(arow, g), blk_off<D>(arow, 2 + g)};
  // Transposing reads (see read_tr): lane (i, G) reads row 4 (G/2) + i/4
  // (+ 8) of the 16-row k-step t, features 16 (G%2) + 4 (i%4) of the
  // 32-feature block db, which is chunk 4 db + 2 (G%2) + (i%4)/2; each (t, db)
  // is one block further.
  const int ti = lane & 15, tG = lane >> 4;
  const int trow0 = 4 * (tG >> 1) + (ti >> 2);
  const int tcl = 2 * (tG & 1) + ((ti & 3) >> 1);
  const int toff_lo = blk_off<D>(trow0, tcl) + 4 * (ti & 1);
  const int toff_hi = blk_off<D>(trow0 + 8, tcl) + 4 * (ti & 1);
  // row records of the lane's rows 8 (r/4) + 4 g + r%4 of the wave's half
  const int rbase = ROLE * 32 + g * 4;

  f32x16 acc[KB][DBLK];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc[kb][db] = f32x16{};
  u32x4 mine[KB][2];   // own P (ROLE 0) or own dS (ROLE 1) of the previous step

  // S[row][key] = Q K^T and dP[row][key] = dO V^T for this wave's 32 rows
  auto scores = [&](int buf, f32x16 (&S)[KB], f32x16 (&dP)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) { S[kb] = f32x16{}; dP[kb] = f32x16{}; }
    const uint16_t* Qb = sm.qd[buf][0];
    const uint16_t* Db = sm.qd[buf][1];
    // operands of k-step ks + 1 are read while the MFMAs of k-step ks run
    u32x4 qa[2], da[2];
    qa[0] = load16(Qb + roff[0]);
    da[0] = load16(Db + roff[0]);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 1 < KSTEPS) {
        const int off = roff[(ks + 1) & 1] + BLK_ELEMS * ((ks + 1) >> 1);
        qa[(ks + 1) & 1] = load16(Qb + off);
        da[(ks + 1) & 1] = load16(Db + off);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        S[kb] = mfma32<T>(qa[ks & 1], kf[kb][ks], S[kb]);
        dP[kb] = mfma32<T>(da[ks & 1], vf[kb][ks], dP[kb]);
      }
    }
  };

  // Stored dS: each wave writes its 32 x 32 block of a step's dS to the image
  // of its row tile and key step, lane (key, g) writing chunks 2 s + g of the
  // block's 32-row column range (see ds_off).  The lane's part of the offset
  // is ds_off(key, g); chunk 2 s + g differs from chunk g by bit 4 of the
  // element offset, and the 32-row range (first row hr, a multiple of 32)
  // selects the block column.
  // Pairs whose keys lie past the sequence's last image store nothing; keys
  // past Lk inside it store zeros (K^T is zero there, and 0 * dS must stay 0).
  const bool ds_on = u.ds >= 0 && u.key0 < u.nks * TILE_ROWS;
  const bool ds_key_ok = u.key0 + l32 < u.Lk;
  const int ds_lane = ds_off((u.key0 & (TILE_ROWS - 1)) + l32, g);
  auto store_ds = [&](int hr, int s, const u32x4& v) {
    uint16_t* img = a.ds + ((int64_t)u.ds + (int64_t)(hr / ROW_TILE) * u.nks + u.key0 / TILE_ROWS) *
                               DS_IMAGE_ELEMS + ((hr & (ROW_TILE - 1)) / 32) * BLK_ELEMS;
    *reinterpret_cast<u32x4*>(img + (ds_lane ^ (16 * s))) = ds_key_ok ? v : u32x4{0u, 0u, 0u, 0u};
  };

  // dropout: gamma times the lane's key (the word of row i and key j is the
  // output function at the row's counter base plus gamma j)
  uint64_t gkey[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) gkey[kb] = SM_GAMMA * (uint64_t)(u.key0 + kb * 32 + l32);

  // window bounds on j - c (an open side: beyond any distance)
  const float wdlo = a.win_left >= 0 ? (float)-a.win_left : -3.0e38f;
  const float wdhi = a.win_right >= 0 ? (float)a.win_right : 3.0e38f;

  // P and dS of the wave's half; the own product's half stays in `mine`, the
  // other goes to the partner through LDS slot `slot`.
  // P and dS of accumulator register r (row rbase + 8 (r/4) + r%4); with
  // dropout P is the kept, scaled weight (dV's operand) and dP is scaled or 0
  auto pointwise = [&](int buf, int r, int r0, f32x16 (&S)[KB], f32x16 (&dP)[KB]) {
    const f32x4 ri = sm.rinfo[buf][rbase + (r >> 2) * 8 + (r & 3)];
    u32x4 dr = u32x4{0u, 0u, 0u, 0u};
    if (DROP) dr = sm.drec[buf][rbase + (r >> 2) * 8 + (r & 3)];
    // WIN: the record holds the unclamped centre c (the bias takes the
    // clamped one) and the row keeps keys j with j - c in [wdlo, wdhi]
    const float cc = WIN ? __builtin_fmaxf(ri[1], 0.0f) : ri[1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float bias = __builtin_fmaf(-ri[0], __builtin_fabsf(cc - keyf[kb]), ri[2]);
      float p, w;
      if (CAP) {
        const float rc = cap_r(S[kb][r], a.lc);
        p = fast_exp2(__builtin_fmaf(a.lc.t_mul, rc, bias));
        w = __builtin_fmaf(-rc, rc, rc);
      } else {
        p = fast_exp2(__builtin_fmaf(S[kb][r], a.lc.s_lin, bias));
        w = 1.0f;
      }
      if (WIN) {
        const float dj = keyf[kb] - ri[1];
        p = dj >= wdlo && dj <= wdhi ? p : 0.0f;
      }
      if (DROP) {
        const bool keep = sm_word_hi(drop_base(dr) + gkey[kb]) >= dr[2];
        const float sc = drop_scale_of(dr);
        const float dpe = keep ? dP[kb][r] * sc : 0.0f;
        dP[kb][r] = p * (dpe - ri[3]) * w;
        S[kb][r] = keep ? p * sc : 0.0f;
      } else {
        S[kb][r] = p;
        dP[kb][r] = p * (dP[kb][r] - ri[3]) * w;
      }
    }
  };
  // packs P and dS; the own product's half goes to `own`, the other to the
  // partner through LDS slot `slot`; dS also to its image
  auto publish = [&](int slot, int r0, f32x16 (&S)[KB], f32x16 (&dP)[KB], u32x4 (&own)[KB][2]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 pb = u32x4{pack2<T>(S[kb][8 * s + 0], S[kb][8 * s + 1]),
                               pack2<T>(S[kb][8 * s + 2], S[kb][8 * s + 3]),
                               pack2<T>(S[kb][8 * s + 4], S[kb][8 * s + 5]),
                               pack2<T>(S[kb][8 * s + 6], S[kb][8 * s + 7])};
        const u32x4 sb = u32x4{pack2<T>(dP[kb][8 * s + 0], dP[kb][8 * s + 1]),
                               pack2<T>(dP[kb][8 * s + 2], dP[kb][8 * s + 3]),
                               pack2<T>(dP[kb][8 * s + 4], dP[kb][8 * s + 5]),
                               pack2<T>(dP[kb][8 * s + 6], dP[kb][8 * s + 7])};
        own[kb][s] = ROLE ? sb : pb;
        sm.xch[slot][wave][kb * 2 + s][lane] = ROLE ? pb : sb;
        if (ds_on) store_ds(r0 + ROLE * 32, s, sb);
      }
  };
  auto pointwise_publish = [&](int buf, int slot, int r0, f32x16 (&S)[KB], f32x16 (&dP)[KB],
                               u32x4 (&own)[KB][2]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) pointwise(buf, r, r0, S, dP);
    publish(slot, r0, S, dP, own);
  };

  // dV (ROLE 0) or dK (ROLE 1) over the 64 rows of a step: A = dO^T or Q^T
  // read transposed from LDS; B = P or dS, from `mine` for the own half and
  // from the partner's slot for the other.  k-step t covers rows 16t .. 16t + 15.
  auto accumulate = [&](int buf, int slot) {
    const uint16_t* X = sm.qd[buf][ROLE ? 0 : 1];
    u32x4 B[KB][2];   // B operands of the partner's half, read up front
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) B[kb][s] = sm.xch[slot][wave ^ 1][kb * 2 + s][lane];
    // the A operand of product i + 1 is read while the MFMAs of product i run
    auto read_a = [&](int i) {
      const int t = i / DBLK, db = i - t * DBLK;
      const int off = (t * (CHUNKS / 4) + db) * BLK_ELEMS;
      const u32x2 lo = read_tr(X + toff_lo + off);
      const u32x2 hi = read_tr(X + toff_hi + off);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 A[2];
    A[0] = read_a(0);
#pragma unroll
    for (int i = 0; i < 4 * DBLK; ++i) {
      if (i + 1 < 4 * DBLK) A[(i + 1) & 1] = read_a(i + 1);
      const int t = i / DBLK, db = i - t * DBLK;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc[kb][db] = mfma32<T>(A[i & 1], (t >> 1) == ROLE ? mine[kb][t & 1] : B[kb][t & 1],
                                acc[kb][db]);
    }
  };

  // visited row steps: every step of a visited tile inside [rb, re) (an
  // empty run leaves the accumulators zero)
  // first step of a visited tile at or after tile t (re when none)
  auto tile_start = [&](int t) {
    t = tile_mask_next(tm, u, t, lane);
    return t > tm.last ? re : max(rb, t * ROW_TILE);
  };
  // the visited step after the one at r0
  auto next_step = [&](int r0) {
    const int r = r0 + KV_ROW_STEP;
    if (r >= re) return re;
    return (r & (ROW_TILE - 1)) != 0 ? r : tile_start(r / ROW_TILE);
  };
  // End of a step: the next step's copies (requested before this step's
  // dS stores, the wave's last 2 KB of vector memory operations) have landed.
  // The stores need not have: nothing in the kernel reads the images.
  auto wait_step_loads = [&]() {
    if (ds_on) wait_vm_le<2 * KB>();
    else wait_vm();
  };
  int rn = rb;   // rows of the step after the current one (the first tile is visited)
  if (rn < re) {
    const int r0 = rn;
    issue_loads(r0, 0);
    rn = next_step(r0);
    wait_vm();
    __syncthreads();
    if (rn < re) issue_loads(rn, 1);
    f32x16 S[KB], dP[KB];
    scores(0, S, dP);
    pointwise_publish(0, 0, r0, S, dP, mine);
    wait_step_loads();
    __syncthreads();
    int prev = 0, cur = 1, next = 2;   // buffers of steps n - 1, n, n + 1
    int n = 1;
    for (; rn < re; ++n) {
      const int rc = rn;
      rn = next_step(rc);
      if (rn < re) issue_loads(rn, next);
      scores(cur, S, dP);
      // products of the previous step (its partner half arrived before the
      // barrier) and the pointwise work of this one are independent; the two
      // waves sharing a SIMD take them in opposite orders, so one runs VALU
      // while the other keeps the matrix core busy
      if (LATE) {
        accumulate(prev, (n - 1) & 1);
        pointwise_publish(cur, n & 1, rc, S, dP, mine);
      } else {
        u32x4 own[KB][2];
        pointwise_publish(cur, n & 1, rc, S, dP, own);
        accumulate(prev, (n - 1) & 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) { mine[kb][0] = own[kb][0]; mine[kb][1] = own[kb][1]; }
      }
      wait_step_loads();
      __syncthreads();
      const int t = prev;
      prev = cur;
      cur = next;
      next = t;
    }
    accumulate(prev, (n - 1) & 1);
  }

  // lane owns key key0 + 32 kb + l32, features 32 db + 8 (r/4) + 4 g + r%4
  const float scale = ROLE ? (CAP ? 4.0f * a.lc.sigma : a.lc.sigma) : 1.0f;
  if (u.part < 0) {
    uint16_t* base = (ROLE ? a.dk : a.dv) + (int64_t)u.kvh * (ROLE ? a.dk_hs : a.dv_hs);
    const int64_t ts = ROLE ? a.dk_ts : a.dv_ts;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = u.key0 + kb * 32 + l32;
      if (key >= u.Lk) continue;
      uint16_t* dst = base + (int64_t)(u.k0 + key) * ts + g * 4;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& A = acc[kb][db];
          *reinterpret_cast<u32x2*>(dst + db * 32 + rq * 8) =
              u32x2{pack2<T>(scale * A[rq * 4 + 0], scale * A[rq * 4 + 1]),
                    pack2<T>(scale * A[rq * 4 + 2], scale * A[rq * 4 + 3])};
        }
    }
  } else {
    float* base = ROLE ? a.part_dk : a.part_dv;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int64_t slot = (int64_t)u.part * KEY_TILE + (u.key0 % KEY_TILE) + kb * 32 + l32;
      float* dst = base + slot * D + g * 4;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& A = acc[kb][db];
          *reinterpret_cast<f32x4*>(dst + db * 32 + rq * 8) =
              f32x4{scale * A[rq * 4 + 0], scale * A[rq * 4 + 1], scale * A[rq * 4 + 2],
                    scale * A[rq * 4 + 3]};
        }
    }
  }
}

}  // namespace kvd

template <class T, int D, bool CAP, bool WIN, bool DROP>
__global__ __launch_bounds__(KV_THREADS, 1) void dkdv_kernel(const AttnArgs a) {
  using namespace kvd;
  __shared__ __attribute__((aligned(16))) KvShared<D, DROP> sm;

  // items [w0, w1) of the work list
  const long long W = a.plan.kv_head[0];
  const int nkt = a.plan.kv_head[1];
  const int seg = a.plan.kv_head[3];
  // Workgroup i runs on XCD i % 8 (round-robin dispatch): it takes share
  // (i % 8) * G / 8 + i / 8, so the shares of one XCD are consecutive and
  // its workgroups walk neighbouring key tiles of the same sequences, whose
  // Q / dO rows then come from that XCD's L2.
  const int G = gridDim.x;
  const int sh = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const long long w0 = (long long)sh * W / G;
  const long long w1 = (long long)(sh + 1) * W / G;
  const int gt0 = a.plan.wg_first[sh];
  if (w0 >= w1 || gt0 < 0) return;
  // Segments in three passes over the share's key tiles: its whole key tiles,
  // then the head of its last one, then the tail of its first one.  Every
  // share thus starts at the first row of a key tile, and since the shares of
  // an XCD hold neighbouring key tiles of the same sequences, its workgroups
  // walk the same Q / dO rows at about the same time and read them through
  // the XCD's L2 (a share that opened with the tail of a key tile would sit
  // at an arbitrary row).  Which segment lands in which partial slot does not
  // change, so neither does any result.
  for (int pass = 0; pass < 3; ++pass)
  for (long long w = w0, gt = gt0; w < w1 && gt < nkt; ++gt) {
    // lane and wave are re-derived per segment behind an empty asm, so the
    // compiler cannot keep the segment's lane-constant offsets live across
    // segments (that pushes the pipeline into scratch)
    int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    asm volatile("" : "+v"(lane), "+v"(wv));
    const int wave = __builtin_amdgcn_readfirstlane(wv);
    const int* e = a.plan.ktab + (int64_t)KV_FIELDS * gt;
    const int V = e[KV_V], S = e[KV_S];
    const long long vs = (long long)S + seg;   // first visit item of the key tile
    if (V == 0 || vs + V <= w) continue;       // nothing of this key tile left
    const long long f = max(w, vs) - vs, l = min(w1, vs + V) - vs;
    if (f >= l) break;   // the share ends among the key tile's segment items
    w = vs + l;
    if ((f > 0 ? 2 : (l < V ? 1 : 0)) != pass) continue;   // whole, head, tail
    const int ktile = e[KV_KTILE];
    KvUnit u;
    u.q0 = e[KV_Q0];
    u.k0 = e[KV_K0];
    u.Lk = e[KV_LK];
    u.rows = e[KV_ROWS];
    u.lq = e[KV_LQ];
    u.lqmul = e[KV_LQMUL];
    u.lqshift = e[KV_LQSHIFT];
    u.hb = e[KV_HB];
    u.kvh = e[KV_G];
    u.rbase = (int64_t)u.q0 * a.hq + (int64_t)u.hb * u.lq;
    u.first = (int)f;
    u.last = (int)l;
    // a key tile split over shares: partial slot 2 sh for the share's first
    // key tile (the share starts at or after the key tile's items), 2 sh + 1
    // for its last
    u.part = (f == 0 && l == V) ? -1 : 2 * sh + (S <= w0 ? 0 : 1);
    u.ds = a.ds ? e[KV_DSOFF] : -1;
    u.nks = (u.Lk + TILE_ROWS - 1) / TILE_ROWS;
    u.ksteps = a.ksteps + 2 * e[KV_RTOFF];
    u.key0 = ktile * KEY_TILE + (wave >> 1) * PAIR_KEYS;
    u.step_lo = ktile * (KEY_TILE / TILE_ROWS);
    // waves w and w + 4 share a SIMD
    if (wave < 4) {
      if (wave & 1) dkdv_wave<T, D, CAP, 1, false, WIN, DROP>(a, sm, u, wave, lane);
      else dkdv_wave<T, D, CAP, 0, false, WIN, DROP>(a, sm, u, wave, lane);
    } else {
      if (wave & 1) dkdv_wave<T, D, CAP, 1, true, WIN, DROP>(a, sm, u, wave, lane);
      else dkdv_wave<T, D, CAP, 0, true, WIN, DROP>(a, sm, u, wave, lane);
    }
    __syncthreads();   // the next segment reuses the LDS buffers
  }
}

template <class T, int D, bool DROP>
static hipError_t launch_dkdv_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  const bool win = a.win_left >= 0 || a.win_right >= 0;
  if (cap) {
    if (win) hipLaunchKernelGGL((dkdv_kernel<T, D, true, true, DROP>), grid, KV_THREADS, 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<T, D, true, false, DROP>), grid, KV_THREADS, 0, s, a);
  } else {
    if (win) hipLaunchKernelGGL((dkdv_kernel<T, D, false, true, DROP>), grid, KV_THREADS, 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<T, D, false, false, DROP>), grid, KV_THREADS, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.drop_on)
    return dtype == DT_BF16 ? launch_dkdv_t<BF16, D, true>(a, cap, grid, s)
                            : launch_dkdv_t<F16, D, true>(a, cap, grid, s);
  return dtype == DT_BF16 ? launch_dkdv_t<BF16, D, false>(a, cap, grid, s)
                          : launch_dkdv_t<F16, D, false>(a, cap, grid, s);
}

}  // namespace rga
