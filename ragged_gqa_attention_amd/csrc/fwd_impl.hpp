// Forward kernel: softmax attention over folded (head, token) rows.
//
// Page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section "What
// You Have": logits are (scale_multiplier / sqrt(D)) q.k, soft-capped to
// c tanh(x / c), shifted by -slope[b,h] |i + Lk - Lq - j|, then softmax-ed over
// the sequence's keys.  Page "python-20261012-ragged-flash-attention-gradient-
// recompute", section "Root causes addressed": stream over key tiles and store
// only O and L = m + log l.
//
// The query heads of a group share one K/V head, so the Lq x group rows of a
// plan sequence (a packed sequence and one K/V head) are folded into one M
// dimension (row = head * Lq + token): a workgroup's 256 rows reuse each
// staged K/V tile 256 times.  The kernels are templated on the head dimension
// D (64, 128 or 160: D / 16 k-steps of the 32x32x16 MFMA); one translation
// unit instantiates each D.  Each wave owns 32 rows and forms
// S^T = K Q^T (keys x rows, Q in registers), so an accumulator lane owns one row
// and O^T = V^T P^T keeps the row scale per lane.  Key steps of 64 are copied
// to LDS with direct loads (three buffers), K and V as row tiles: S^T reads
// its K operand with one 16-byte read per MFMA, P V its V^T operand with two
// transposing reads (ds_read_b64_tr_b16), so the forward needs no transposed
// copy of V.
//
// Softmax offset.  Distances are measured from the clamped centre
// c_i = max(i + Lk - Lq, 0): for a row with i + Lk - Lq < 0 every key lies to
// its right, so |i + Lk - Lq - j| = j + dmin_i with dmin_i = Lq - Lk - i, and the
// constant slope * dmin_i moves into the row offset
//   m_i = c - slope * dmin_i   (capped; without a cap, -slope * dmin_i).
// With a cap every logit of row i is at most m_i, so m_i is used as the softmax
// offset fixed before the key loop: P = exp(a - m) <= 1, the nearest key keeps
// P >= e^{-2c}, and no running maximum, rescale or cross-lane max is needed
// (the normalised result is the same as with the true maximum).  Without a cap
// a running maximum relative to m_i is kept.  The row statistic is stored as
// L = m_i + log l (natural log) and, for the backward, as the small residual
// log2 l relative to m_i, so the backward never subtracts two large numbers.
// The backward's per-row record (slope, centre, residual, Delta) is written
// here in the full-VJP call, Delta = rowsum(dO * O) taken from the FP32 O.
//
// Far keys.  With a cap, a key farther from a row's centre than the skip
// bound allows has P == 0 exactly (see row_key_steps), so a workgroup visits
// only the key steps [lo, hi) that hold a key some row of its tile keeps (the
// planner records that range per tile).  In the full-VJP call one more
// workgroup plans the dK/dV units meanwhile.
#pragma once

#include "dropout.hpp"
#include "kernels.hpp"
#include "planner.hpp"
#include "tiles.hpp"

namespace rga {

// LDS of a key step: the K and V rows (row tiles, blk_off), three buffers
// (one step in flight, one being read, and, with dropout, the previous one
// still read by the deferred half of waves 4-7; the O staging of the
// epilogue needs their room in any case).
constexpr int FWD_NBUF = 3;
template <int D>
struct FwdShared {
  uint16_t k[FWD_NBUF][tile_elems<D>()];
  uint16_t v[FWD_NBUF][tile_elems<D>()];
};
// After the key loop the same LDS holds the normalised O rows (pitch of D + 8
// elements) and each row's record.
template <int D> constexpr int o_pitch() { return D + 8; }

// Grid: workgroup 0 runs the planner (then, in the full-VJP call, the dK/dV
// unit plan), workgroups 1 .. a.fwd_slots the row tiles.  The row tiles do
// not wait for the planner: each finds its tile and key-step range from
// cu_q / cu_k itself (find_row_tile, tile_key_range), so the planner runs
// beside them on one compute unit.
// One 256-row tile of the forward: sequence b (extents q0, Lq, k0, Lk), tile
// `tile` of its folded rows, key steps [klo, khi).
template <class T, int D, bool CAP, bool DELTA, bool WIN, bool DROP>
__device__ __forceinline__ void fwd_tile(const AttnArgs& a, FwdShared<D>& sm, const int b,
                                         const int tile, const int q0, const int Lq,
                                         const int k0, const int Lk, const int klo,
                                         const int khi, int* const grab = nullptr,
                                         int* const grabbed = nullptr, const int grab_base = 0) {
  constexpr int KSTEPS = Geo<D>::KSTEPS, DBLK = Geo<D>::DBLK, CHUNKS = Geo<D>::CHUNKS;
  constexpr int BLK_COLS = Geo<D>::BLK_COLS, O_PITCH = o_pitch<D>();
  static_assert(ROW_TILE * O_PITCH * 2 + ROW_TILE * 16 <= (int)sizeof(FwdShared<D>),
                "O staging fits the key-tile buffers");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int rows = Lq * a.group;
  // plan sequence b = packed sequence bp, K/V head kvh (query heads hb ..)
  const int bp = b / a.hkv, kvh = b - bp * a.hkv, hb = kvh * a.group;
  const uint16_t* kbase = a.k + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + (int64_t)kvh * a.v_hs;

  // copies of key step kt: waves 0-3 the K rows, waves 4-7 the V rows (one
  // 16-row group each).  Rows past Lk repeat row Lk - 1 (the tile runs before
  // the planner has cleared the zero block): only the last, masked step has
  // them, where their logits are -inf, so they add 0 * (a finite V row).
  // Issued unseen by the compiler (it would hold the step's transposing reads
  // until the next step's copies had landed); advance() orders the buffers.
  // The first step's copies go out before the Q rows are requested.
  const uint16_t* klast = kbase + (int64_t)(k0 + max(Lk, 1) - 1) * a.k_ts;
  const uint16_t* vlast = vbase + (int64_t)(k0 + max(Lk, 1) - 1) * a.v_ts;
  auto issue = [&](int kt, int buf) {
    if (wave < 4)
      load_row_tile<D, true>(sm.k[buf], kbase + (int64_t)k0 * a.k_ts, a.k_ts, kt * TILE_ROWS,
                             Lk, klast, wave, lane);
    else
      load_row_tile<D, true>(sm.v[buf], vbase + (int64_t)k0 * a.v_ts, a.v_ts, kt * TILE_ROWS,
                             Lk, vlast, wave - 4, lane);
  };
  if (klo < khi) issue(klo, klo % FWD_NBUF);

  const int row = tile * ROW_TILE + wave * 32 + l32;
  const bool row_ok = row < rows;
  const int rr = row_ok ? row : rows - 1;
  // folded row -> (token, head): R = h * Lq + i (two divisions per workgroup)
  const int hh = rr / Lq, ti = rr - hh * Lq;

  // Q row as B operand: k-step ks covers features 16ks + 8g .. +7
  const uint16_t* qrow = a.q + (int64_t)(q0 + ti) * a.q_ts + (int64_t)(hb + hh) * a.q_hs + g * 8;
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = load16(qrow + ks * 16);

  const float slope2 = a.slopes[(int64_t)bp * a.slopes_stride + hb + hh] * LOG2E;
  // key j of accumulator register r in block kb of the tile at kbase is
  // kbase + 32 kb + 8 (r/4) + 4 g + r%4; cb0 - (kbase + 32 kb + 8 (r/4) + r%4)
  // is then j's signed distance from the clamped centre max(i + Lk - Lq, 0)
  const float cb0 = (float)(max(ti + Lk - Lq, 0) - 4 * g);
  // window (WIN): the row keeps keys [wlo, whi), bounds around its unclamped
  // centre i + Lk - Lq; a row keeping none ends with l = 0 (out 0, L = -inf)
  const int wc = ti + Lk - Lq;
  const int wlo = WIN && a.win_left >= 0 ? wc - a.win_left : 0;
  const int whi = WIN && a.win_right >= 0 ? min(Lk, wc + a.win_right + 1) : Lk;
  // the wave's tightest bounds: blocks inside [wlo_max, whi_min) are unmasked
  int wlo_max = wlo, whi_min = whi;
  if (WIN) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      wlo_max = max(wlo_max, __shfl_xor(wlo_max, o, 64));
      whi_min = min(whi_min, __shfl_xor(whi_min, o, 64));
    }
    wlo_max = __builtin_amdgcn_readfirstlane(wlo_max);
    whi_min = __builtin_amdgcn_readfirstlane(whi_min);
  }
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)max(0, Lq - Lk - ti);
  // log2 units, relative to moff.  With a cap, the largest exponent a kept key
  // can reach: 0 for slope >= 0 (the nearest kept key is the clamped centre
  // itself), and -slope2 times the largest distance from the clamped centre to
  // a kept key for a negative slope, which favours far keys.
  float m = -__builtin_inff();
  if (CAP) {
    m = 0.0f;
    if (slope2 < 0.0f) {
      const int cc = max(ti + Lk - Lq, 0);
      const int jlo = max(wlo, 0), jhi = max(whi, jlo + 1);
      m = -slope2 * (float)max(abs(cc - jlo), abs(cc - (jhi - 1)));
    }
  }
  const float negm = CAP ? -m : 0.0f;
  float lsum = 0.0f;     // exact sum of P
  float lsum_r = 0.0f;   // sum of P rounded to the input dtype
  f32x16 O[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) O[db] = f32x16{};

  const int ntiles = (Lk + TILE_ROWS - 1) / TILE_ROWS;

  // lane-constant LDS offsets: K row reads (row kb * 32 + l32, chunk 2 ks + g)
  // and transposing V reads (see read_tr): lane (i, G) addresses key rows
  // 4 (G/2) + i/4 and + 8 of a 16-key k-step, chunk 2 (G%2) + (i%4)/2 of a
  // 32-feature block, the low or high half of its 16 bytes by i % 2
  const int koff[2] = {blk_off<D>(l32, g), blk_off<D>(l32, 2 + g)};
  const int vi = lane & 15, vG = lane >> 4;
  const int vrow = 4 * (vG >> 1) + (vi >> 2);
  const int vcl = 2 * (vG & 1) + ((vi & 3) >> 1);
  const int voff_lo = blk_off<D>(vrow, vcl) + 4 * (vi & 1);
  const int voff_hi = blk_off<D>(vrow + 8, vcl) + 4 * (vi & 1);

  // S^T[key][row] = K Q^T (lane = row) for key block kb of the K tile Kb
  // (LDS operands are read two k-steps ahead of the MFMA that uses them)
  f32x16 S[2];
  auto scores = [&](int kb, const uint16_t* Kb) {
    const uint16_t* Kr = Kb + kb * 2 * BLK_COLS * BLK_ELEMS;
    auto kop = [&](int ks) { return load16(Kr + koff[ks & 1] + (ks >> 1) * BLK_ELEMS); };
    u32x4 ka[3];
    ka[0] = kop(0);
    ka[1] = kop(1);
    S[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 2 < KSTEPS) ka[(ks + 2) % 3] = kop(ks + 2);
      S[kb] = mfma32<T>(ka[ks % 3], qf[ks], S[kb]);
    }
  };
  // capped and biased logits (log2 units) of key block kb of the step at
  // kbase; masked: keys past Lk get -inf (only a partial last step needs it,
  // the compare and select cost a VALU pair per logit)
  // near: the step holds keys on both sides of some row's centre; otherwise
  // (every key at or before every centre of the wave) the distance is
  // cb - jl >= 0 and the bias slope2 jl - slope2 cb + negm takes one FMA
  // per logit instead of a subtraction and an FMA.  The two forms differ by
  // the rounding of slope2 cb, below 2^-23 (150 + 64 slope2) for any logit
  // whose weight does not underflow.
  auto logits = [&](int kb, int kbase, auto masked, auto near) {
    const float cb = cb0 - (float)kbase;
    const float cl = __builtin_fmaf(-slope2, cb, negm);
    const int kleft = whi - kbase - 4 * g;         // keys of this lane group still in range
    const int kfrom = wlo - kbase - 4 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jl = kb * 32 + (r >> 2) * 8 + (r & 3);
      // (the order of the two only steers the register allocator: cap first
      // spills least in the dropout instances, bias first runs fastest in
      // the others)
      float rc = 0.0f, bias;
      auto bias_of = [&]() {
        return decltype(near)::value
                   ? __builtin_fmaf(-slope2, __builtin_fabsf(cb - (float)jl), negm)
                   : __builtin_fmaf(slope2, (float)jl, cl);
      };
      if (DROP) {
        if (CAP) rc = cap_r(S[kb][r], a.lc);
        bias = bias_of();
      } else {
        bias = bias_of();
        if (CAP) rc = cap_r(S[kb][r], a.lc);
      }
      float x;
      if (CAP)
        x = __builtin_fmaf(a.lc.t_mul, rc, bias);
      else if (decltype(near)::value)
        x = __builtin_fmaf(-slope2, __builtin_fabsf(cb - (float)jl), S[kb][r] * a.lc.s_lin);
      else
        x = __builtin_fmaf(S[kb][r], a.lc.s_lin, bias);
      if (!WIN && decltype(masked)::value) x = jl < kleft ? x : -__builtin_inff();
      S[kb][r] = x;
    }
    // WIN: only a block that some row's window cuts (or that reaches past
    // Lk, where every window ends) pays for the per-logit test
    if (WIN) {
      const int j0 = kbase + kb * 32;
      if (!(j0 >= wlo_max && j0 + 32 <= whi_min)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = kb * 32 + (r >> 2) * 8 + (r & 3);
          S[kb][r] = jl >= kfrom && jl < kleft ? S[kb][r] : -__builtin_inff();
        }
      }
    }
  };
  // P rounded to the input dtype feeds the PV product, and O is normalised by
  // the sum of those same rounded values (lsum_r), so O is an exact convex
  // combination of V rows: a single-key row reproduces v_0 and delta = dO.O
  // matches dP.  L and the backward's residual use the exact FP32 sum.
  // Dropout: the row's record (counter base, threshold, scale); the sums l
  // and lsum_r stay those of the undropped weights, the PV operand holds the
  // kept ones and the scale multiplies O at the end.
  u32x4 drec = u32x4{0u, 0u, 0u, 0u};
  uint64_t dbase = 0;
  if (DROP) {
    drec = drop_row(a, bp, hb + hh, ti, (int64_t)(q0 + ti));
    dbase = drop_base(drec) + SM_GAMMA * (uint64_t)(4 * g);   // this lane's key offset 4 g
  }
  u32x4 pb[2][2];
  auto probs = [&](int kb, int kbase) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(S[kb][r]);
      lsum += p;
      S[kb][r] = p;
    }
    auto pack = [&]() {
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pb[kb][s] = u32x4{pack2<T>(S[kb][8 * s + 0], S[kb][8 * s + 1]),
                          pack2<T>(S[kb][8 * s + 2], S[kb][8 * s + 3]),
                          pack2<T>(S[kb][8 * s + 4], S[kb][8 * s + 5]),
                          pack2<T>(S[kb][8 * s + 6], S[kb][8 * s + 7])};
    };
    pack();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 4; ++w) lsum_r = add_pair<T>(pb[kb][s][w], lsum_r);
    if (DROP) {
      const uint64_t zs = dbase + SM_GAMMA * (uint64_t)kbase;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t jl = kb * 32 + (r >> 2) * 8 + (r & 3);
        if (!drop_keep(zs, jl, drec[2])) S[kb][r] = 0.0f;
      }
      pack();
    }
  };
  // O^T[d][row] += V^T[d][keys] P^T[keys][row] for key block kb of the V row
  // tile Vb; product i = 2 db + s takes features 32 db .. + 31 and the
  // 16-key k-step 2 kb + s, read transposed in the key order of pb
  auto pv = [&](int kb, const uint16_t* Vb) {
    auto vop = [&](int i) {
      const int off = ((2 * kb + (i & 1)) * BLK_COLS + (i >> 1)) * BLK_ELEMS;
      const u32x2 lo = read_tr(Vb + voff_lo + off);
      const u32x2 hi = read_tr(Vb + voff_hi + off);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 va[3];
    va[0] = vop(0);
    va[1] = vop(1);
#pragma unroll
    for (int i = 0; i < 2 * DBLK; ++i) {
      if (i + 2 < 2 * DBLK) va[(i + 2) % 3] = vop(i + 2);
      O[i >> 1] = mfma32<T>(va[i % 3], pb[kb][i & 1], O[i >> 1]);
    }
  };

  // tile kt has landed for every wave, and every wave is done with kt - 2;
  // then start the copies of kt + 1 (three buffers)
  auto advance = [&](int kt) {
    wait_vm();
    __syncthreads();
    if (kt + 1 < khi) issue(kt + 1, (kt + 1) % FWD_NBUF);
  };
  // the key mask costs a compare and a select per logit, so only a partial
  // last key step runs the masked instance (after the loop); steps
  // [klo, kfull) are full ones
  const int nfull = Lk / TILE_ROWS;
  const bool partial = nfull < ntiles && khi == ntiles;
  const int kfull = min(khi, nfull);
  constexpr Flag<false> unmasked{};
  constexpr Flag<true> masked{};
  // far steps [klo, kfar): every key lies at or before every clamped centre
  // of the wave's rows (see logits); they come first, then the near ones.
  // (With dropout every step takes the general form: the dropout variant is
  // already short of registers and a second loop body pushes it to spill.)
  int kfar = klo;
  if (!DROP) {
    int cmin = max(ti + Lk - Lq, 0);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) cmin = min(cmin, __shfl_xor(cmin, o, 64));
    kfar = min(kfull, (__builtin_amdgcn_readfirstlane(cmin) + 1) / TILE_ROWS);
  }

  if (CAP) {
    // The offset is fixed, so the two 32-key blocks of a step are
    // independent: every wave takes a step as S0 S1 | logits/P 0 | PV0 |
    // logits/P 1 | PV1.  (Offsetting the two waves of a SIMD, one of them
    // deferring block 1 of each step into the next, measured 1.5 % slower.)
    // (b1 false: every key of block 1 lies past Lk, so its weights are
    // exactly 0 and add nothing to O or l; only a partial last step has it)
    auto step = [&](int kt, auto mk, auto nr, bool b1 = true) {
      const int buf = kt % FWD_NBUF, kbase = kt * TILE_ROWS;
      scores(0, sm.k[buf]);
      if (b1) scores(1, sm.k[buf]);
      logits(0, kbase, mk, nr);
      probs(0, kbase);
      pv(0, sm.v[buf]);
      if (b1) {
        logits(1, kbase, mk, nr);
        probs(1, kbase);
        pv(1, sm.v[buf]);
      }
    };
    // With dropout, waves w and w + 4 (one SIMD) run offset instead: wave
    // w + 4 defers block 1 of each step into the next (it reads the previous
    // step's V tile, hence three LDS buffers); under the dropout variant's
    // register pressure that order spills least.
    auto run_drop = [&](auto lag) {
      constexpr bool LAG = decltype(lag)::value;
      auto step1 = [&](int kt, auto mk) {
        const int buf = kt % FWD_NBUF, kbase = kt * TILE_ROWS;
        if (LAG && kt > klo) {   // the previous step is a full one
          logits(1, kbase - TILE_ROWS, Flag<WIN>{}, Flag<true>{});
          probs(1, kbase - TILE_ROWS);
          pv(1, sm.v[(kt - 1) % FWD_NBUF]);
        }
        scores(0, sm.k[buf]);
        scores(1, sm.k[buf]);
        logits(0, kbase, mk, Flag<true>{});
        probs(0, kbase);
        pv(0, sm.v[buf]);
        if (!LAG) {
          logits(1, kbase, mk, Flag<true>{});
          probs(1, kbase);
          pv(1, sm.v[buf]);
        }
      };
      for (int kt = klo; kt < kfull; ++kt) {
        advance(kt);
        step1(kt, unmasked);
      }
      if (partial) {
        advance(nfull);
        step1(nfull, masked);
      }
      if (LAG && klo < khi) {   // block 1 of the last step
        const int kt = khi - 1;
        if (partial) logits(1, kt * TILE_ROWS, masked, Flag<true>{});
        else logits(1, kt * TILE_ROWS, unmasked, Flag<true>{});
        probs(1, kt * TILE_ROWS);
        pv(1, sm.v[kt % FWD_NBUF]);
      }
    };
    if (DROP) {
      if (wave < 4) run_drop(Flag<false>{});
      else run_drop(Flag<true>{});
    } else {
      int kt = klo;
      for (; kt < kfar; ++kt) {
        advance(kt);
        step(kt, unmasked, Flag<false>{});
      }
      for (; kt < kfull; ++kt) {
        advance(kt);
        step(kt, unmasked, Flag<true>{});
      }
      if (partial) {
        advance(nfull);
        step(nfull, masked, Flag<true>{}, Lk - nfull * TILE_ROWS > 32);
      }
    }
  } else {
    // running maximum over both blocks of a step, then rescale
    auto step = [&](int kt, auto mk, auto nr) {
      const int buf = kt % FWD_NBUF, kbase = kt * TILE_ROWS;
      scores(0, sm.k[buf]);
      scores(1, sm.k[buf]);
      logits(0, kbase, mk, nr);
      logits(1, kbase, mk, nr);
      float tmax = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = __builtin_fmaxf(tmax, S[kb][r]);
      tmax = __builtin_fmaxf(tmax, swap_half(tmax));
      const float mnew = __builtin_fmaxf(m, tmax);
      // a windowed row may see only masked keys so far: subtract 0, not -inf
      const float msub = WIN && mnew == -__builtin_inff() ? 0.0f : mnew;
      const float alpha = fast_exp2(m - msub);
      m = mnew;
      lsum *= alpha;
      lsum_r *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) O[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kb][r] -= msub;
      probs(0, kbase);
      probs(1, kbase);
      pv(0, sm.v[buf]);
      pv(1, sm.v[buf]);
    };
    int kt = klo;
    if (!DROP)
      for (; kt < kfar; ++kt) {
        advance(kt);
        step(kt, unmasked, Flag<false>{});
      }
    for (; kt < kfull; ++kt) {
      advance(kt);
      step(kt, unmasked, Flag<true>{});
    }
    if (partial) {
      advance(nfull);
      step(nfull, masked, Flag<true>{});
    }
  }

  // grab (ticket dealing): the workgroup's next rank is requested here, so the
  // atomic's round trip overlaps the epilogue, and lands in *grabbed at the end
  int ticket_got = 0;
  if (grab != nullptr && threadIdx.x == 0) ticket_got = atomicAdd(grab, 1);
  // Epilogue.  The normalised O goes through LDS so that global stores (and
  // the dO loads of Delta) move whole 64-byte pieces of rows: in the
  // accumulator layout a lane holds 8-byte pieces of one row, which would
  // touch a new row every lane.  Delta = dO . O uses the rounded O, as the
  // standalone backward does from the stored output (plus, with dropout, the
  // rounding residual, see below).
  // lanes 4q .. 4q + 3 of wave w later take row 32 w + 16 h + q (h = 0, 1),
  // chunks (lane % 4) + 4 i; their dO pieces are requested first
  int erow[2];
  bool eok[2];
  uint16_t* eout[2];
  u32x4 dpre[2][CHUNKS / 4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rg = tile * ROW_TILE + wave * 32 + 16 * h + (lane >> 2);
    erow[h] = rg;
    eok[h] = rg < rows;
    const int rc = eok[h] ? rg : rows - 1;
    const int hd = rc / Lq, tk = rc - hd * Lq;
    eout[h] = a.out + (int64_t)(q0 + tk) * a.o_ts + (int64_t)(hb + hd) * a.o_hs;
    if (DELTA) {
      const uint16_t* drow =
          a.dout + (int64_t)(q0 + tk) * a.do_ts + (int64_t)(hb + hd) * a.do_hs;
#pragma unroll
      for (int i = 0; i < CHUNKS / 4; ++i) dpre[h][i] = load16(drow + ((lane & 3) + 4 * i) * 8);
    }
  }
  lsum += swap_half(lsum);
  lsum_r += swap_half(lsum_r);
  const float inv = lsum_r > 0.0f ? (DROP ? drop_scale_of(drec) : 1.0f) / lsum_r
                                  : 0.0f;
  const float res = m + fast_log2(lsum);
  __syncthreads();   // every wave is done with the key tiles
  uint16_t* obuf = reinterpret_cast<uint16_t*>(&sm);
  f32x4* sinfo = reinterpret_cast<f32x4*>(obuf + ROW_TILE * O_PITCH);
  const int lrow = wave * 32 + l32;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *reinterpret_cast<u32x2*>(obuf + lrow * O_PITCH + db * 32 + rq * 8 + g * 4) =
          u32x2{pack2<T>(O[db][rq * 4 + 0] * inv, O[db][rq * 4 + 1] * inv),
                pack2<T>(O[db][rq * 4 + 2] * inv, O[db][rq * 4 + 3] * inv)};
  if (g == 0) {
    sinfo[lrow] = f32x4{slope2, (float)(WIN ? ti + Lk - Lq : max(ti + Lk - Lq, 0)),
                        lsum > 0.0f ? -res : 0.0f, 0.0f};
    // the backward's dropout record of this row
    if (DELTA && DROP && row_ok)
      a.droprec[(int64_t)q0 * a.hq + (int64_t)hb * Lq + row] = drec;
    if (row_ok)
      a.lse[(int64_t)(q0 + ti) * a.hq + hb + hh] =
          lsum > 0.0f ? (moff + res) * LN2 : -__builtin_inff();
  }
  __syncthreads();
  float dpart[2] = {0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 32 + 16 * h + (lane >> 2);
    const bool ok = eok[h];
#pragma unroll
    for (int i = 0; i < CHUNKS / 4; ++i) {
      const int c = (lane & 3) + 4 * i;
      const u32x4 o = load16(obuf + r * O_PITCH + c * 8);
      if (ok) *reinterpret_cast<u32x4*>(eout[h] + c * 8) = o;
      if (DELTA) {
        const u32x4 d = dpre[h][i];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dpart[h] += lo_f<T>(o[e]) * lo_f<T>(d[e]) + hi_f<T>(o[e]) * hi_f<T>(d[e]);
      }
    }
  }
  if (DELTA && DROP) {
    // With dropout, O carries the scale 1 / (1 - p), so the rounded output no
    // longer reproduces the FP32 dP of a row with a single kept key exactly:
    // Delta adds dO . (O - round(O)), the residual staged through the same
    // LDS rows, which brings it to the FP32 O.
    __syncthreads();   // every wave has read its rounded rows
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float o = O[db][rq * 4 + e] * inv;
          const uint32_t w = pack2<T>(o, 0.0f);
          x[e] = o - lo_f<T>(w);
        }
        *reinterpret_cast<u32x2*>(obuf + lrow * O_PITCH + db * 32 + rq * 8 + g * 4) =
            u32x2{pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3])};
      }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = wave * 32 + 16 * h + (lane >> 2);
#pragma unroll
      for (int i = 0; i < CHUNKS / 4; ++i) {
        const u32x4 o = load16(obuf + r * O_PITCH + ((lane & 3) + 4 * i) * 8);
        const u32x4 d = dpre[h][i];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dpart[h] += lo_f<T>(o[e]) * lo_f<T>(d[e]) + hi_f<T>(o[e]) * hi_f<T>(d[e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 32 + 16 * h + (lane >> 2);
    const int rg = erow[h];
    const bool ok = eok[h];
    if (DELTA) {
      dpart[h] += __shfl_xor(dpart[h], 1, 64);
      dpart[h] += __shfl_xor(dpart[h], 2, 64);
    }
    if (ok && (lane & 3) == 0 && a.rowinfo) {
      f32x4 rec = sinfo[r];
      rec[3] = DELTA ? dpart[h] : 0.0f;
      *reinterpret_cast<f32x4*>(a.rowinfo + ((int64_t)q0 * a.hq + (int64_t)hb * Lq + rg) * 4) =
          rec;
    }
  }
  if (grab != nullptr && threadIdx.x == 0) *grabbed = grab_base + ticket_got;
}

// The forward's row tiles in a fixed order: plan sequences by key length,
// longest first (ties by index), for up to 64 of them, else batch order; each
// workgroup builds the table of that order once (from cu_q / cu_k alone).
constexpr int FWD_ORDER_MAX = 512;
struct FwdOrder {
  int status;   // 1: table, 2: too many sequences (find_row_tile per rank), 0: nothing
  int n, nrt;
  int start[FWD_ORDER_MAX + 1];   // first rank of entry k; start[n] = nrt
  int seq[FWD_ORDER_MAX], q0[FWD_ORDER_MAX], lq[FWD_ORDER_MAX], k0[FWD_ORDER_MAX],
      lk[FWD_ORDER_MAX];
  int lqv[64], lkv[64];   // query / key lengths by plan sequence (up to 64 of them)
  int part[16];   // block scan partials
};

template <int NT>
__device__ __forceinline__ void build_fwd_order(const PlanArgs& pa, FwdOrder& ord) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = pa.batch, hq = pa.hq;   // plan sequences, rows folded per sequence
  if (B <= 64) {
    if (wave == 0) {
      const int b = lane;
      const bool live = b < B;
      // B >= 1: the forward is not launched otherwise
      const SeqExt e = seq_extents(pa, min(b, B - 1));
      const bool any_bad = __any(live && e.bad);
      const int lq = live ? e.nq - e.cq : 0, lk = live ? e.nk - e.ck : 0;
      const int n = live ? (lq * hq + ROW_TILE - 1) / ROW_TILE : 0;
      int start = 0, rank = 0;   // over the sequences ranked before b
      for (int j = 0; j < B; ++j) {
        const int lkj = __builtin_amdgcn_readlane(lk, j), nj = __builtin_amdgcn_readlane(n, j);
        const bool before = lkj > lk || (lkj == lk && j < b);
        start += before ? nj : 0;
        rank += before ? 1 : 0;
      }
      int total = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) total += __shfl_xor(total, o, 64);
      if (live) {
        ord.start[rank] = start;
        ord.seq[rank] = b;
        ord.q0[rank] = e.cq;
        ord.lq[rank] = lq;
        ord.k0[rank] = e.ck;
        ord.lk[rank] = lk;
        ord.lqv[b] = lq;
        ord.lkv[b] = lk;
      }
      if (lane == 0) {
        ord.start[B] = total;
        ord.n = B;
        ord.nrt = total;
        ord.status = any_bad ? 0 : 1;
      }
    }
  } else if (B <= FWD_ORDER_MAX) {
    bool bad = false;
    for (int b = tid; b < B; b += NT) {
      const SeqExt e = seq_extents(pa, b);
      bad |= e.bad;
      ord.seq[b] = b;
      ord.q0[b] = e.cq;
      ord.lq[b] = max(e.nq - e.cq, 0);
      ord.k0[b] = e.ck;
      ord.lk[b] = max(e.nk - e.ck, 0);
    }
    const bool any_bad = __syncthreads_or(bad);
    block_exclusive_scan<NT>(B, [&](int b) { return (ord.lq[b] * hq + ROW_TILE - 1) / ROW_TILE; },
                             [&](int b, int v) { ord.start[b] = v; }, ord.part);
    if (tid == 0) {
      ord.n = B;
      ord.nrt = ord.start[B];
      ord.status = any_bad ? 0 : 1;
    }
  } else if (tid == 0) {
    ord.status = 2;
  }
  __syncthreads();
}

// Longest-first ranks.  For batches of up to 64 sequences, 4096 (sequence,
// head) pairs and 2048 row tiles, each persistent workgroup also ranks every
// tile by its key steps (longest first, ties in table order: every workgroup
// derives the same ranking) and resolves the ranks it deals itself before its
// first tile; the snake then pairs long tiles with short ones.  The scratch
// lives in the key-tile buffers, which no tile uses yet.
constexpr int LPT_CLASSES = 1024;   // key steps (longer tiles share class 0)
constexpr int LPT_SPER = LPT_MAX_HEADS / ROW_THREADS;   // slopes per thread
struct LptScratch {
  int hlo[LPT_MAX_HEADS];         // key-step range of every token of (plan sequence, head)
  int hhi[LPT_MAX_HEADS];
  int hw[LPT_MAX_HEADS];          // key half-width of (plan sequence, head)
  int cls[LPT_MAX_TILES];         // class of tile t (t: rank in table order)
  int ks[LPT_MAX_TILES][2];       // key-step range of tile t
  int hist[LPT_CLASSES];
  int off[LPT_CLASSES + 1];       // first rank of each class
};

// Fills list[i] = {b, tile, q0, lq, k0, lk, klo, khi} for the workgroup's
// ranks r < nrt (round i of the snake); returns their count, or -1 when the
// batch does not qualify (the caller then finds each tile itself).
// Whether lpt_list ranks this batch (its scratch holds every (plan sequence,
// head) and every tile), and its slopes, requested by the caller before the
// sequence table so that the two loads overlap: thread tid holds (plan
// sequence, head) pairs tid, tid + NT, ... in plan-sequence order.
__device__ __forceinline__ bool lpt_fits(const PlanArgs& pa) {
  return pa.batch <= LPT_MAX_SEQS && pa.batch * pa.hq <= LPT_MAX_HEADS;
}
template <int NT>
__device__ __forceinline__ void lpt_load_slopes(const PlanArgs& pa, float (&sv)[LPT_SPER]) {
  const int hq = pa.hq, n = pa.batch * hq;
#pragma unroll
  for (int i = 0; i < LPT_SPER; ++i) {
    const int p = (int)threadIdx.x + i * NT;
    sv[i] = 0.0f;
    if (i * NT < n && p < n) {
      const int v = p / hq;
      sv[i] = pa.slopes[slope_base(v, pa.hkv, hq, pa.slopes_stride) + (p - v * hq)];
    }
  }
}

template <int NT>
__device__ __forceinline__ int lpt_list(const PlanArgs& pa, const FwdOrder& ord, LptScratch& sc,
                                        int (*list)[8], int w, int P,
                                        const float (&sv)[LPT_SPER]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = pa.batch, hq = pa.hq, nrt = ord.nrt;
  if (!lpt_fits(pa) || nrt > LPT_MAX_TILES) return -1;
  // rounds of the snake; a workgroup's ranks grow from round to round, so it
  // stops at its first rank past the last tile
  const int rounds = (nrt + P - 1) / P;
  if (rounds > FWD_LIST_MAX) return -1;
  // half-width and whole-head key-step range of every (plan sequence, head)
  for (int c = tid; c < LPT_CLASSES; c += NT) sc.hist[c] = 0;
#pragma unroll
  for (int i = 0; i < LPT_SPER; ++i) {
    const int p = tid + i * NT;
    if (i * NT < B * hq && p < B * hq) {
      const int v = p / hq, lq = ord.lqv[v], lk = ord.lkv[v];
      const int hw = key_half_width(sv[i] * LOG2E, lk, pa.skip_log2);
      sc.hw[p] = hw;
      int l = 0x7fffffff, u = 0;
      if (lq > 0) token_range_steps(0, lq - 1, lq, lk, hw, pa.win_left, pa.win_right, l, u);
      sc.hlo[p] = l;
      sc.hhi[p] = u;
    }
  }
  __syncthreads();
  auto entry_of = [&](int t) {   // last table entry whose first rank is <= t
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ord.start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int t = tid; t < nrt; t += NT) {   // tile_key_steps of every tile
    const int k = entry_of(t);
    const int lq = ord.lq[k], lk = ord.lk[k];
    const int hbase = ord.seq[k] * hq;
    const int R0 = (t - ord.start[k]) * ROW_TILE, R1 = min(lq * hq, R0 + ROW_TILE);
    const int hfirst = R0 / lq, hlast = (R1 - 1) / lq;
    int lo = 0x7fffffff, hi = 0;
    // the first and last heads may hold part of their tokens; the ones
    // between hold all of them (the whole-head range)
    for (int h = hfirst; h <= hlast; ++h) {
      int l, u;
      if (h == hfirst || h == hlast) {
        const int ia = h == hfirst ? R0 - h * lq : 0;
        const int ib = h == hlast ? R1 - 1 - h * lq : lq - 1;
        token_range_steps(ia, ib, lq, lk, sc.hw[hbase + h], pa.win_left, pa.win_right, l, u);
      } else {
        l = sc.hlo[hbase + h];
        u = sc.hhi[hbase + h];
      }
      if (l < u) {
        lo = min(lo, l);
        hi = max(hi, u);
      }
    }
    finish_range(lo, hi);
    const int c = LPT_CLASSES - 1 - min(max(hi - lo, 0), LPT_CLASSES - 1);
    sc.cls[t] = c;
    sc.ks[t][0] = lo;
    sc.ks[t][1] = hi;
    atomicAdd(&sc.hist[c], 1);
  }
  __syncthreads();
  if (wave == 0) {   // class offsets: lane l scans classes 16 l .. 16 l + 15
    constexpr int CPL = LPT_CLASSES / 64;
    int sum = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) sum += sc.hist[lane * CPL + i];
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    int run = x - sum;
    for (int i = 0; i < CPL; ++i) {
      sc.off[lane * CPL + i] = run;
      run += sc.hist[lane * CPL + i];
    }
    if (lane == 63) sc.off[LPT_CLASSES] = run;
  }
  __syncthreads();
  // each wave resolves some of the workgroup's ranks (round i falls to wave
  // i % 8): the class c of rank r is the last class with off <= r (a search
  // over 64 and then 16 offsets, each one ballot), then the tile is the
  // (r - off[c])-th of class c in table order
  int n = 0;   // rounds whose rank lies below nrt (a prefix: ranks grow)
  for (int round = 0; round < rounds; ++round)
    if (round * P + ((round & 1) ? P - 1 - w : w) < nrt) n = round + 1;
  for (int round = wave; round < n; round += NT / 64) {
    const int r = round * P + ((round & 1) ? P - 1 - w : w);
    constexpr int CPL = LPT_CLASSES / 64;
    const uint64_t b1 = __ballot(sc.off[lane * CPL] <= r);   // lane 0's offset is 0
    const int L = 63 - __builtin_clzll(b1);
    const uint64_t b2 = __ballot(lane < CPL && sc.off[L * CPL + min(lane, CPL - 1)] <= r);
    const int c = L * CPL + (63 - __builtin_clzll(b2));
    int want = r - sc.off[c], t = -1;
    for (int base = 0; base < nrt && t < 0; base += 64) {
      const uint64_t m = __ballot(base + lane < nrt && sc.cls[base + lane] == c);
      const int cnt = __popcll(m);
      if (want < cnt) {
        uint64_t mm = m;
        for (int i = 0; i < want; ++i) mm &= mm - 1;   // drop the lowest want bits
        t = base + __builtin_ctzll(mm);
      } else {
        want -= cnt;
      }
    }
    // table entry of tile t: the last with start <= t
    const uint64_t be = __ballot(lane < B && ord.start[min(lane, B - 1)] <= t);
    const int k = 63 - __builtin_clzll(be);
    if (lane == 0) {
      list[round][0] = ord.seq[k];
      list[round][1] = t - ord.start[k];
      list[round][2] = ord.q0[k];
      list[round][3] = ord.lq[k];
      list[round][4] = ord.k0[k];
      list[round][5] = ord.lk[k];
      list[round][6] = sc.ks[t][0];
      list[round][7] = sc.ks[t][1];
    }
  }
  return n;   // the same in every thread; list[] is complete after a barrier
}

// Seat of worker workgroup j (1 <= j < G) at the snake's table: the workers
// of XCD 0 first, then those of XCD 1, and so on.  Workgroup j runs on XCD
// j % 8 (the dispatcher deals workgroups round robin), so the consecutive
// ranks of a round (the row tiles of one sequence sit next to each other in
// the ranking) go to one XCD and share its L2 for their K and V rows.
__device__ __forceinline__ int worker_seat(int j, int G) {
  const int x = j & 7;
  int before = 0;   // workers j' >= 1 with j' % 8 < x
  for (int y = 0; y < x; ++y) before += (y < G ? (G - y + 7) / 8 : 0) - (y == 0 ? 1 : 0);
  return before + (j >> 3) - (x == 0 ? 1 : 0);
}

// Grid: workgroup 0 runs the planner (then, in the full-VJP call, the dK/dV
// unit plan); workgroups 1 .. P (one per remaining compute unit) are
// persistent and deal the row tiles among themselves like cards in a snake:
// in round r the worker at seat w (worker_seat) takes rank r P + w (r even)
// or r P + P - 1 - w (r odd), so a workgroup whose first tile was among the
// longest takes one of the shortest next.  The row tiles never wait for the planner: a workgroup
// finds each tile and its key-step range from cu_q / cu_k itself (the order
// table, tile_key_range), so the planner runs beside them.
// LDS of the forward grid: the key-step buffers of the row tiles, or the
// planner's tables (workgroup 0), or the longest-first ranking scratch that a
// row-tile workgroup uses before its first tile.
template <int D>
union FwdSmem {
  FwdShared<D> f;
  PlanShared p;
  UnitsShared u;
  LptScratch l;
};

template <class T, int D, bool CAP, bool DELTA, bool WIN, bool DROP>
__global__ __launch_bounds__(ROW_THREADS, 1) void fwd_kernel(const AttnArgs a, const PlanArgs pa) {
  __shared__ __attribute__((aligned(16))) FwdSmem<D> smu;
  __shared__ FwdOrder ord;
  __shared__ int tinfo[8];
  FwdShared<D>& sm = smu.f;

  if (blockIdx.x == 0) {
    plan_block<ROW_THREADS>(pa, smu.p);
    if (DELTA) {   // the full-VJP call: the dK/dV units, from the planner's ranges
      __syncthreads();
      plan_units<ROW_THREADS>(pa, a.plan.seq, smu.u);
    }
    return;
  }
  const int w = worker_seat((int)blockIdx.x, (int)gridDim.x), P = (int)gridDim.x - 1;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float sv[LPT_SPER];
  if (lpt_fits(pa)) lpt_load_slopes<ROW_THREADS>(pa, sv);
  build_fwd_order<ROW_THREADS>(pa, ord);
  const int status = ord.status;
  if (status == 0) return;
  // longest-first: the workgroup's tiles resolved in advance (nlist >= 0)
  __shared__ int list[FWD_LIST_MAX][8];
  __shared__ int nlist_s;
  if (status == 1) {
    const int n = lpt_list<ROW_THREADS>(pa, ord, smu.l, list, w, P, sv);
    if (threadIdx.x == 0) nlist_s = n;
  } else if (threadIdx.x == 0) {
    nlist_s = -1;
  }
  __syncthreads();
  const int nlist = nlist_s;
  if (nlist >= 0) {
    for (int i = 0; i < nlist; ++i) {
      fwd_tile<T, D, CAP, DELTA, WIN, DROP>(a, sm, list[i][0], list[i][1], list[i][2], list[i][3],
                                      list[i][4], list[i][5], list[i][6], list[i][7]);
      __syncthreads();   // the next tile reuses the LDS buffers
    }
    return;
  }
  // Without the ranked list, rank r is the r-th tile of the order table (or
  // of batch order).  Round 0 deals ranks 0 .. P - 1 by seat; after that a
  // workgroup that finishes a tile takes the next rank from the ticket
  // (a.fwd_ticket, reset before the launch), so the tiles of large batches,
  // whose lengths the snake cannot pair up, go to whichever workgroup is free
  // first.  Without a ticket the snake continues.  Every rank is taken once
  // either way, and a tile's result does not depend on who computes it.
  // (The dropout instances keep the snake: the ticket code pushes their
  // register allocation into spills.)  Each tile requests the next rank
  // during its epilogue (fwd_tile), so the atomic's round trip stays off the
  // path.  (One ticket per XCD, keeping a sequence's neighbouring tiles in one
  // L2, balanced worse and measured slower at three of four such workloads.)
  int* const ticket = DROP ? nullptr : a.fwd_ticket;
  __shared__ int next_rank;
  for (int round = 0;; ++round) {
    const bool by_ticket = ticket != nullptr && round > 0;
    const int r = by_ticket ? next_rank : round * P + ((round & 1) ? P - 1 - w : w);
    if (!by_ticket && status == 1 && r >= ord.nrt) break;
    // wave 0 finds the tile of rank r and its key steps (the planner's
    // range) and hands them over through LDS
    if (wave == 0) {
      RowTile rt{};
      bool ok = true;
      if (status == 1 && r >= ord.nrt) {
        ok = false;
      } else if (status == 1) {   // last table entry whose first rank is <= r (a nonempty one)
        int lo = 0, hi = ord.n - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (ord.start[mid] <= r) lo = mid; else hi = mid - 1;
        }
        rt.b = ord.seq[lo];
        rt.tile = r - ord.start[lo];
        rt.q0 = ord.q0[lo];
        rt.lq = ord.lq[lo];
        rt.k0 = ord.k0[lo];
        rt.lk = ord.lk[lo];
      } else {
        ok = find_row_tile(pa, r, rt);
      }
      int klo = 0, khi = 0;
      if (ok) tile_key_range(pa, rt, klo, khi);
      if (lane == 0) {
        tinfo[0] = ok ? rt.b : -1;
        tinfo[1] = rt.tile;
        tinfo[2] = rt.q0;
        tinfo[3] = rt.lq;
        tinfo[4] = rt.k0;
        tinfo[5] = rt.lk;
        tinfo[6] = klo;
        tinfo[7] = khi;
      }
    }
    __syncthreads();
    const int b = tinfo[0];
    if (b < 0) break;
    fwd_tile<T, D, CAP, DELTA, WIN, DROP>(a, sm, b, tinfo[1], tinfo[2], tinfo[3], tinfo[4], tinfo[5],
                                    tinfo[6], tinfo[7], ticket, &next_rank, P);
    __syncthreads();   // the next tile reuses tinfo and the LDS buffers
  }
}


template <class T, int D, bool WIN, bool DROP>
static hipError_t launch_fwd_t(const AttnArgs& a, const PlanArgs& pa, bool cap, bool with_delta,
                               int grid, hipStream_t s) {
  if (cap) {
    if (with_delta)
      hipLaunchKernelGGL((fwd_kernel<T, D, true, true, WIN, DROP>), grid, ROW_THREADS, 0, s, a,
                         pa);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, true, false, WIN, DROP>), grid, ROW_THREADS, 0, s, a,
                         pa);
  } else {
    if (with_delta)
      hipLaunchKernelGGL((fwd_kernel<T, D, false, true, WIN, DROP>), grid, ROW_THREADS, 0, s, a,
                         pa);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, false, false, WIN, DROP>), grid, ROW_THREADS, 0, s, a,
                         pa);
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd_td(const AttnArgs& a, const PlanArgs& pa, bool cap, bool with_delta,
                                int grid, hipStream_t s) {
  const bool win = a.win_left >= 0 || a.win_right >= 0;
  if (a.drop_on)
    return win ? launch_fwd_t<T, D, true, true>(a, pa, cap, with_delta, grid, s)
               : launch_fwd_t<T, D, false, true>(a, pa, cap, with_delta, grid, s);
  return win ? launch_fwd_t<T, D, true, false>(a, pa, cap, with_delta, grid, s)
             : launch_fwd_t<T, D, false, false>(a, pa, cap, with_delta, grid, s);
}

template <int D>
hipError_t launch_fwd_d(const AttnArgs& a, const PlanArgs& pa, int dtype, bool cap,
                        bool with_delta, hipStream_t s) {
  // the planner plus one persistent workgroup per remaining compute unit
  const int grid = 1 + max(1, a.kv_wgs - 1);
  if (a.batch <= 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_fwd_td<BF16, D>(a, pa, cap, with_delta, grid, s)
                          : launch_fwd_td<F16, D>(a, pa, cap, with_delta, grid, s);
}

}  // namespace rga
