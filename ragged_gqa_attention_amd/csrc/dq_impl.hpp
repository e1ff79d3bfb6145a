// dQ kernel: recompute P and dP per row tile from the stored row record, then
//   dS = P * (dP - Delta) * (1 - tanh^2(s / c)),  dQ = sigma dS K.
//
// Page "python-20261012-ragged-flash-attention-gradient-recompute", section
// "Root causes addressed": no probability matrix is stored; the backward
// rebuilds each tile from L.  Page "Noncausal Global Extreme-GQA Ragged
// Attention Full VJP", section "Hard Constraints": the cap sits between the
// scaled dot product and ALiBi, so its derivative multiplies dP - Delta.
//
// With r = 1 / (1 + e^{2s/c}), 1 - tanh^2(s/c) = 4 r (1 - r); the kernel forms
// r - r^2 and folds the factor 4 into the final sigma scale.
//
// P is rebuilt exactly as the forward formed it: distances from the clamped
// centre max(i + Lk - Lq, 0), the large per-row offset kept analytic, and only
// the small residual log2 l subtracted (see fwd.hip), so no two large numbers
// are ever subtracted.  Templated on the head dimension D (64, 128, 160); one
// translation unit per D.
//
// A workgroup owns 256 folded rows (like the forward) and walks the keys in
// steps of 64, copied to LDS with direct loads (double-buffered): K and V as
// row tiles; S^T and dP^T read their K / V operand with one 16-byte read per
// MFMA, dQ^T its K^T operand with two transposing reads of the K rows.  It visits only the key
// steps the forward recorded for the tile (a.ksteps): outside them every P,
// and so every dS, is exactly zero.
#pragma once

#include "dropout.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

namespace dqd {

// LDS of one key step: K and V rows (row tiles, blk_off), double-buffered.
template <int D>
struct DqShared {
  uint16_t k[2][tile_elems<D>()];
  uint16_t v[2][tile_elems<D>()];
};

// dK / dV of the 128-key tiles part, part + parts, ... (batch order): key
// tiles whose visits fell to several dK/dV workgroups (see plan_units) sum
// the FP32 partials of those workgroups in workgroup order and round once;
// key tiles no row tile visits (e.g. every key of a sequence without query
// rows) get exact zeros; the others were stored by their one workgroup.  The
// dK/dV kernel has finished (same stream), so its partials are complete.  A
// tile is 128 x 40 groups of 4 features, ten per thread, whose sums are
// formed side by side (ten loads per tensor in flight).
template <class T, int D>
__device__ __forceinline__ void reduce_kv_tiles(const AttnArgs& a, int part, int parts) {
  constexpr int QUADS = D / 4;
  constexpr int PER_THREAD = KEY_TILE * QUADS / ROW_THREADS;
  static_assert(PER_THREAD * ROW_THREADS == KEY_TILE * QUADS, "whole tiles per pass");
  const long long W = a.plan.kv_head[0];
  const int nkt = a.plan.kv_head[1];
  const int seg = a.plan.kv_head[3];
  const long long G = a.kv_wgs;
  for (int gt = part; gt < nkt; gt += parts) {
    const int* e = a.plan.ktab + (int64_t)KV_FIELDS * gt;
    const int V = e[KV_V];
    const long long S = e[KV_S];
    // workgroups holding its first and last visit items, S + seg and
    // S + seg + V - 1: the one whose share [p W / G, (p + 1) W / G) contains
    // item x is p = ((x + 1) G - 1) / W
    int pa = 0, pb = -1;
    if (V > 0) {
      const long long vs = S + seg;
      pa = (int)(((vs + 1) * G - 1) / W);
      pb = (int)(((vs + V) * G - 1) / W);
      if (pa == pb) continue;   // stored by its one workgroup
    }
    const int k0 = e[KV_K0] + e[KV_KTILE] * KEY_TILE;
    const int nkeys = min(KEY_TILE, e[KV_LK] - e[KV_KTILE] * KEY_TILE);
    uint16_t* dkb = a.dk + (int64_t)e[KV_G] * a.dk_hs;
    uint16_t* dvb = a.dv + (int64_t)e[KV_G] * a.dv_hs;
    f32x4 sk[PER_THREAD], sv[PER_THREAD];
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      sk[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      sv[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int p = pa; p <= pb; ++p) {
      const long long p0 = (long long)p * W / G, p1 = (long long)(p + 1) * W / G;
      if (p0 >= p1) continue;   // an empty share wrote nothing
      const int64_t slot = 2 * (int64_t)p + (S <= p0 ? 0 : 1);
      const float* pk = a.part_dk + slot * KEY_TILE * D;
      const float* pv = a.part_dv + slot * KEY_TILE * D;
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) {
        const int i = threadIdx.x + j * ROW_THREADS;   // key i / 40, features 4 (i % 40)
        sk[j] += *reinterpret_cast<const f32x4*>(pk + 4 * i);
        sv[j] += *reinterpret_cast<const f32x4*>(pv + 4 * i);
      }
    }
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int i = threadIdx.x + j * ROW_THREADS;
      const int key = i / QUADS, c4 = i - key * QUADS;
      if (key >= nkeys) continue;
      const int64_t t = k0 + key;
      *reinterpret_cast<u32x2*>(dkb + t * a.dk_ts + c4 * 4) =
          u32x2{pack2<T>(sk[j][0], sk[j][1]), pack2<T>(sk[j][2], sk[j][3])};
      *reinterpret_cast<u32x2*>(dvb + t * a.dv_ts + c4 * 4) =
          u32x2{pack2<T>(sv[j][0], sv[j][1]), pack2<T>(sv[j][2], sv[j][3])};
    }
  }
}

// Stores the dQ accumulators of a 256-row tile.  The rounded values go
// through LDS (row pitch 168 elements, reusing the tile buffers after a
// barrier) so that each global store writes 64-byte pieces of rows: lanes
// 4q .. 4q + 3 of wave w take row 32 w + 16 h + q, chunks (lane % 4) + 4 i.
// lrow: the tile-local row the lane's accumulator column belongs to.
template <class T, int D>
__device__ __forceinline__ void store_dq_tile(const AttnArgs& a, uint16_t* stage,
                                              const f32x16 (&dQ)[Geo<D>::DBLK], float scale,
                                              int lrow, int tile, const int* sq, int wave,
                                              int lane) {
  constexpr int DBLK = Geo<D>::DBLK, CHUNKS = Geo<D>::CHUNKS;
  const int q0 = sq[SQ_Q0], rows = sq[SQ_ROWS];
  constexpr int PITCH = D + 8;
  const int g = lane >> 5;
  __syncthreads();   // every wave is done with the tile buffers
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *reinterpret_cast<u32x2*>(stage + lrow * PITCH + db * 32 + rq * 8 + g * 4) =
          u32x2{pack2<T>(scale * dQ[db][rq * 4 + 0], scale * dQ[db][rq * 4 + 1]),
                pack2<T>(scale * dQ[db][rq * 4 + 2], scale * dQ[db][rq * 4 + 3])};
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 32 + 16 * h + (lane >> 2);
    const int rg = tile * ROW_TILE + r;
    if (rg >= rows) continue;
    int tk, hd;
    unfold_row(rg, sq, tk, hd);
    uint16_t* drow = a.dq + (int64_t)(q0 + tk) * a.dq_ts + (int64_t)(sq[SQ_HB] + hd) * a.dq_hs;
#pragma unroll
    for (int i = 0; i < CHUNKS / 4; ++i) {
      const int c = (lane & 3) + 4 * i;
      *reinterpret_cast<u32x4*>(drow + c * 8) = load16(stage + r * PITCH + c * 8);
    }
  }
}

// LDS of the stored-dS path: the dS image (64 keys x 256 rows, ds_off) and
// the K rows (blk_off) of a key step, three buffers (two steps in flight).
constexpr int DQS_NBUF = 3;
template <int D>
struct DqStoredShared {
  uint16_t ds[DQS_NBUF][DS_IMAGE_ELEMS];
  uint16_t k[DQS_NBUF][tile_elems<D>()];
};
static_assert(ROW_TILE * (160 + 8) <= DQS_NBUF * DS_IMAGE_ELEMS, "dQ staging fits");

// dQ of row tile `tile` from the dS images the dK/dV kernel stored:
// dQ^T[d][row] += K^T[d][keys] dS^T[keys][row], nothing recomputed.  Both
// operands come from LDS with two transposing reads each: K^T from the K rows,
// dS^T from the image (lane l32 gets row 32 w + tt_key_pos(l32), keys in the
// order of the K^T read).  Limited by the HBM reads of the images.
// The first two steps' copies are issued before the workgroup's slice of
// the dK / dV partial sums, so they land while it runs.
template <class T, int D, bool CAP>
__device__ __forceinline__ void dq_stored(const AttnArgs& a, DqStoredShared<D>& sm, const int* sq,
                                          int tile, int klo, int khi) {
  constexpr int DBLK = Geo<D>::DBLK, BLK_COLS = Geo<D>::BLK_COLS;
  const int q0 = sq[SQ_Q0], Lk = sq[SQ_LK], rows = sq[SQ_ROWS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int nks = (Lk + TILE_ROWS - 1) / TILE_ROWS;
  const uint16_t* img0 = a.ds + ((int64_t)sq[SQ_DSOFF] + (int64_t)tile * nks) * DS_IMAGE_ELEMS;
  const int k0 = sq[SQ_K0];
  const uint16_t* kbase = a.k + (int64_t)sq[SQ_G] * a.k_hs;
  // copies of key step kt: each wave four 1 KB blocks of the image, waves 0-3
  // also a 16-row group of the K rows (D / 32 loads: 4 + D / 32 or 4 per wave)
  constexpr int IMG_LOADS = DS_IMAGE_ELEMS / BLK_ELEMS / ROW_WAVES;
  static_assert(IMG_LOADS == 4, "waits below count 4 image loads per wave and step");
  // (issued unseen by the compiler, which would otherwise hold each step's
  // transposing reads until the copies of the two steps ahead had landed;
  // the waits below order the buffers)
  auto issue = [&](int kt, int buf) {
    const uint16_t* img = img0 + (int64_t)kt * DS_IMAGE_ELEMS;
#pragma unroll
    for (int j = 0; j < IMG_LOADS; ++j) {
      const int blk = IMG_LOADS * wave + j;
      load_lds16_unseen(img + blk * BLK_ELEMS + lane * 8, sm.ds[buf] + blk * BLK_ELEMS);
    }
    if (wave < 4)
      load_row_tile<D, true>(sm.k[buf], kbase + (int64_t)k0 * a.k_ts, a.k_ts, kt * TILE_ROWS, Lk,
                             a.zero, wave, lane);
  };

  // transposing reads (see read_tr): lane (i, G) addresses key rows
  // 4 (G/2) + i/4 and + 8 of k-step t, chunk 4 w + 2 (G%2) + (i%4)/2
  const int ti = lane & 15, tG = lane >> 4;
  const int krow = 4 * (tG >> 1) + (ti >> 2);
  const int chunk = 4 * wave + 2 * (tG & 1) + ((ti & 3) >> 1);
  const int dlo = ds_off(krow, chunk) + 4 * (ti & 1);
  const int dhi = ds_off(krow + 8, chunk) + 4 * (ti & 1);
  constexpr int KSTEP_ELEMS = (ROW_TILE / 32) * BLK_ELEMS;   // 16 keys of an image
  // K^T operand: transposing reads of the K row tile in the same key order
  // (lane (i, G): key rows 4 (G/2) + i/4 and + 8 of the k-step, chunk
  // 2 (G%2) + (i%4)/2 of the feature block, half i % 2)
  const int kcl = 2 * (tG & 1) + ((ti & 3) >> 1);
  const int koff_lo = blk_off<D>(krow, kcl) + 4 * (ti & 1);
  const int koff_hi = blk_off<D>(krow + 8, kcl) + 4 * (ti & 1);

  f32x16 dQ[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dQ[db] = f32x16{};
  // (klo <= khi: every range leaves the planner through finish_range)
  if (klo < khi) issue(klo, klo % DQS_NBUF);
  if (klo + 1 < khi) issue(klo + 1, (klo + 1) % DQS_NBUF);
  for (int kt = klo; kt < khi; ++kt) {
    const int buf = kt % DQS_NBUF;
    // step kt has landed (step kt + 1 may still be in flight) for every wave,
    // and every wave is done with step kt - 1, whose buffer step kt + 2 takes
    if (kt + 1 < khi) {
      if (wave < 4) wait_vm_le<IMG_LOADS + BLK_COLS>();
      else wait_vm_le<IMG_LOADS>();
    } else {
      wait_vm();
    }
    __syncthreads();
    if (kt + 2 < khi) issue(kt + 2, (kt + 2) % DQS_NBUF);
    const uint16_t* Ds = sm.ds[buf];
    const uint16_t* Kb = sm.k[buf];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x2 lo = read_tr(Ds + dlo + t * KSTEP_ELEMS);
      const u32x2 hi = read_tr(Ds + dhi + t * KSTEP_ELEMS);
      const u32x4 bt = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int off = (t * BLK_COLS + db) * BLK_ELEMS;
        const u32x2 klo2 = read_tr(Kb + koff_lo + off);
        const u32x2 khi2 = read_tr(Kb + koff_hi + off);
        dQ[db] = mfma32<T>(u32x4{klo2[0], klo2[1], khi2[0], khi2[1]}, bt, dQ[db]);
      }
    }
  }

  // lane l32 holds row 32 w + tt_key_pos(l32) of the tile
  store_dq_tile<T, D>(a, sm.ds[0], dQ, CAP ? 4.0f * a.lc.sigma : a.lc.sigma,
                      wave * 32 + tt_key_pos(l32), tile, sq, wave, lane);
}

template <int D>
union DqSmem {
  DqShared<D> r;
  DqStoredShared<D> d;
};

}  // namespace dqd

template <class T, int D, bool CAP, bool WIN, bool DROP>
__global__ __launch_bounds__(ROW_THREADS, 1) void dq_kernel(const AttnArgs a) {
  using namespace dqd;
  constexpr int KSTEPS = Geo<D>::KSTEPS, DBLK = Geo<D>::DBLK, BLK_COLS = Geo<D>::BLK_COLS;
  __shared__ __attribute__((aligned(16))) DqSmem<D> sm;

  // The grid holds the row-tile slots plus R workgroups that sum the split
  // dK / dV partials, a slice each; those come right after the first round
  // of row tiles (one per compute unit), so they run while the longest tiles
  // do instead of lengthening the tail.
  const int R = (int)gridDim.x - a.fwd_slots;
  const int nrt = a.batch > 0 ? a.plan.kv_head[2] : 0;   // row tiles
  const int at = min(nrt, a.kv_wgs);
  if ((int)blockIdx.x >= at && (int)blockIdx.x < at + R) {
    if (a.total_k > 0) reduce_kv_tiles<T, D>(a, blockIdx.x - at, R);
    return;
  }
  const int slot = (int)blockIdx.x < at ? (int)blockIdx.x : (int)blockIdx.x - R;
  const int b = a.plan.fwd_map[2 * slot];
  if (b < 0) return;
  const int tile = a.plan.fwd_map[2 * slot + 1];
  const int* sq = a.plan.seq + b * SEQ_FIELDS;
  const int* ks = a.ksteps + 2 * (sq[SQ_RTOFF] + tile);
  const int klo = ks[0], khi = ks[1];
  if (a.ds && sq[SQ_DSOFF] >= 0) {
    dq_stored<T, D, CAP>(a, sm.d, sq, tile, klo, khi);
    return;
  }
  const int q0 = sq[SQ_Q0], k0 = sq[SQ_K0], Lk = sq[SQ_LK];
  const int rows = sq[SQ_ROWS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int row = tile * ROW_TILE + wave * 32 + l32;
  const bool row_ok = row < rows;
  const int rr = row_ok ? row : rows - 1;
  int ti, hh;
  unfold_row(rr, sq, ti, hh);
  const int hb = sq[SQ_HB];
  // folded row record (rows of the group's heads follow q0 hq + hb Lq)
  const int64_t ri = (int64_t)q0 * a.hq + (int64_t)hb * sq[SQ_LQ] + rr;

  const uint16_t* qrow = a.q + (int64_t)(q0 + ti) * a.q_ts + (int64_t)(hb + hh) * a.q_hs + g * 8;
  const uint16_t* dorow =
      a.dout + (int64_t)(q0 + ti) * a.do_ts + (int64_t)(hb + hh) * a.do_hs + g * 8;
  const uint16_t* kbase = a.k + (int64_t)sq[SQ_G] * a.k_hs;
  const uint16_t* vbase = a.v + (int64_t)sq[SQ_G] * a.v_hs;
  u32x4 qf[KSTEPS], df[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = load16(qrow + ks * 16);
    df[ks] = load16(dorow + ks * 16);
  }
  // row record: slope * log2(e), centre (unclamped under a window), -residual,
  // Delta
  const f32x4 info = Lk > 0 ? *reinterpret_cast<const f32x4*>(a.rowinfo + ri * 4)
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float slope2 = info[0];
  const float cb0 = (WIN ? __builtin_fmaxf(info[1], 0.0f) : info[1]) - (float)(4 * g);
  const float boff = info[2];
  const float dl = info[3];
  // dropout record of the row: counter base (plus this lane's key offset
  // 4 g), threshold, scale; dP of a dropped key is 0, of a kept one scaled
  u32x4 drec = u32x4{0u, 0u, 0u, 0u};
  uint64_t dbase = 0;
  if (DROP) {
    drec = Lk > 0 && row_ok ? a.droprec[ri] : u32x4{0u, 0u, 0u, 0u};
    dbase = drop_base(drec) + SM_GAMMA * (uint64_t)(4 * g);
  }
  // window (WIN): the row keeps keys [wlo, whi) around its unclamped centre
  const int wc = ti + Lk - sq[SQ_LQ];
  const int wlo = WIN && a.win_left >= 0 ? wc - a.win_left : 0;
  const int whi = WIN && a.win_right >= 0 ? min(Lk, wc + a.win_right + 1) : Lk;

  f32x16 dQ[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dQ[db] = f32x16{};

  const int ntiles = (Lk + TILE_ROWS - 1) / TILE_ROWS;
  // copies of key step kt (40 wave loads): waves 0-3 a 16-row group of K,
  // waves 4-7 one of V; issued unseen by the compiler (advance() orders the
  // buffers before the transposing reads of K)
  auto issue = [&](int kt, int buf) {
    if (wave < 4)
      load_row_tile<D, true>(sm.r.k[buf], kbase + (int64_t)k0 * a.k_ts, a.k_ts, kt * TILE_ROWS,
                             Lk, a.zero, wave, lane);
    else
      load_row_tile<D, true>(sm.r.v[buf], vbase + (int64_t)k0 * a.v_ts, a.v_ts, kt * TILE_ROWS,
                             Lk, a.zero, wave - 4, lane);
  };

  // lane-constant LDS offsets: K / V row reads (row kb * 32 + l32, chunk
  // 2 ks + g) and transposing K reads for the K^T operand (lane (i, G): key
  // rows 4 (G/2) + i/4 and + 8 of a k-step, chunk 2 (G%2) + (i%4)/2, half i % 2)
  const int koff[2] = {blk_off<D>(l32, g), blk_off<D>(l32, 2 + g)};
  const int vi = lane & 15, vG = lane >> 4;
  const int trow = 4 * (vG >> 1) + (vi >> 2), tcl = 2 * (vG & 1) + ((vi & 3) >> 1);
  const int toff_lo = blk_off<D>(trow, tcl) + 4 * (vi & 1);
  const int toff_hi = blk_off<D>(trow + 8, tcl) + 4 * (vi & 1);

  // one key step on the tiles in LDS buffer buf; masked: keys past Lk get P = 0
  auto step = [&](int buf, int kbase, auto masked) {
    const uint16_t* Kb = sm.r.k[buf];
    const uint16_t* Vb = sm.r.v[buf];
    const float cb = cb0 - (float)kbase;
    const int kleft = whi - kbase - 4 * g;
    const int kfrom = wlo - kbase - 4 * g;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T[key][row] = K Q^T and dP^T[key][row] = V dO^T (lane = row)
      f32x16 S = f32x16{}, dP = f32x16{};
      const int rb = kb * 2 * BLK_COLS * BLK_ELEMS;   // rows kb * 32 ..
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int off = koff[ks & 1] + (ks >> 1) * BLK_ELEMS + rb;
        S = mfma32<T>(load16(Kb + off), qf[ks], S);
        dP = mfma32<T>(load16(Vb + off), df[ks], dP);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = kb * 32 + (r >> 2) * 8 + (r & 3);
        const float bias = __builtin_fmaf(-slope2, __builtin_fabsf(cb - (float)jl), boff);
        float p, w;
        if (CAP) {
          const float rc = cap_r(S[r], a.lc);
          p = fast_exp2(__builtin_fmaf(a.lc.t_mul, rc, bias));
          w = __builtin_fmaf(-rc, rc, rc);
        } else {
          p = fast_exp2(__builtin_fmaf(S[r], a.lc.s_lin, bias));
          w = 1.0f;
        }
        if (WIN) p = jl >= kfrom && jl < kleft ? p : 0.0f;
        else if (decltype(masked)::value) p = jl < kleft ? p : 0.0f;
        if (DROP) {
          const bool keep = drop_keep(dbase + SM_GAMMA * (uint64_t)kbase, (uint32_t)jl, drec[2]);
          const float dpe = keep ? dP[r] * drop_scale_of(drec) : 0.0f;
          S[r] = p * (dpe - dl) * w;
        } else {
          S[r] = p * (dP[r] - dl) * w;
        }
      }
      u32x4 sb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        sb[s] = u32x4{pack2<T>(S[8 * s + 0], S[8 * s + 1]), pack2<T>(S[8 * s + 2], S[8 * s + 3]),
                      pack2<T>(S[8 * s + 4], S[8 * s + 5]), pack2<T>(S[8 * s + 6], S[8 * s + 7])};
      // dQ^T[d][row] += K^T[d][keys] dS^T[keys][row]; the K^T operand is two
      // transposing reads of the K rows, in the key order of sb
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int off = ((2 * kb + s) * BLK_COLS + db) * BLK_ELEMS;
          const u32x2 lo = read_tr(Kb + toff_lo + off);
          const u32x2 hi = read_tr(Kb + toff_hi + off);
          dQ[db] = mfma32<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, sb[s], dQ[db]);
        }
    }
  };

  // tile kt has landed for every wave, and every wave is done with kt - 1;
  // then start the copies of kt + 1
  auto advance = [&](int kt) {
    wait_vm();
    __syncthreads();
    if (kt + 1 < khi) issue(kt + 1, (kt + 1) & 1);
  };
  // the key mask costs a compare and a select per logit, so only a partial
  // last key step runs the masked instance (after the loop)
  const int nfull = Lk / TILE_ROWS;
  if (klo < khi) issue(klo, klo & 1);
  for (int kt = klo; kt < min(khi, nfull); ++kt) {
    advance(kt);
    step(kt & 1, kt * TILE_ROWS, Flag<false>{});
  }
  if (nfull < ntiles && khi == ntiles) {
    advance(nfull);
    step(nfull & 1, nfull * TILE_ROWS, Flag<true>{});
  }

  store_dq_tile<T, D>(a, sm.r.k[0], dQ, CAP ? 4.0f * a.lc.sigma : a.lc.sigma, wave * 32 + l32,
                      tile, sq, wave, lane);
}

template <class T, int D, bool DROP>
static hipError_t launch_dq_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  const bool win = a.win_left >= 0 || a.win_right >= 0;
  if (cap) {
    if (win) hipLaunchKernelGGL((dq_kernel<T, D, true, true, DROP>), grid, ROW_THREADS, 0, s, a);
    else hipLaunchKernelGGL((dq_kernel<T, D, true, false, DROP>), grid, ROW_THREADS, 0, s, a);
  } else {
    if (win) hipLaunchKernelGGL((dq_kernel<T, D, false, true, DROP>), grid, ROW_THREADS, 0, s, a);
    else hipLaunchKernelGGL((dq_kernel<T, D, false, false, DROP>), grid, ROW_THREADS, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.drop_on)
    return dtype == DT_BF16 ? launch_dq_t<BF16, D, true>(a, cap, grid, s)
                            : launch_dq_t<F16, D, true>(a, cap, grid, s);
  return dtype == DT_BF16 ? launch_dq_t<BF16, D, false>(a, cap, grid, s)
                          : launch_dq_t<F16, D, false>(a, cap, grid, s);
}

}  // namespace rga
