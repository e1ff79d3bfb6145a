// Forward kernel: softmax attention over folded (head, token) rows.
//
// Page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section "What
// You Have": logits are (scale_multiplier / sqrt(D)) q.k, soft-capped to
// c tanh(x / c), shifted by -slope[b,h] |i + Lk - Lq - j|, then softmax-ed over
// the sequence's keys.  Page "python-20261012-ragged-flash-attention-gradient-
// recompute", section "Root causes addressed": stream over key tiles and store
// only O and L = m + log l.
//
// Every query head shares the one K/V head, so the Lq x Hq rows of a sequence
// are folded into one M dimension (row = head * Lq + token): a workgroup's 256
// rows reuse each staged K/V tile 256 times.  Each wave owns 32 rows and forms
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
#include "kernels.hpp"
#include "planner.hpp"
#include "tiles.hpp"

namespace rga {

namespace {

// LDS of a key step: the K and V rows (row tiles, blk_off), three buffers
// (one step in flight, one being read, and the previous one still read by the
// deferred half of the lag waves).
constexpr int FWD_NBUF = 3;
struct FwdShared {
  uint16_t k[FWD_NBUF][TILE_ELEMS];
  uint16_t v[FWD_NBUF][TILE_ELEMS];
};
// After the key loop the same LDS holds the normalised O rows (pitch of 168
// elements) and each row's record.
constexpr int O_PITCH = HEAD_DIM + 8;
static_assert(ROW_TILE * O_PITCH * 2 + ROW_TILE * 16 <= (int)sizeof(FwdShared),
              "O staging fits the key-tile buffers");

}  // namespace

static_assert(sizeof(UnitsShared) <= sizeof(FwdShared), "the unit planner fits the tile buffers");
static_assert(sizeof(PlanShared) <= sizeof(FwdShared), "the planner fits the tile buffers");

// Grid: workgroup 0 runs the planner (then, in the full-VJP call, the dK/dV
// unit plan), workgroups 1 .. a.fwd_slots the row tiles.  The row tiles do
// not wait for the planner: each finds its tile and key-step range from
// cu_q / cu_k itself (find_row_tile, tile_key_range), so the planner runs
// beside them on one compute unit.
template <class T, bool CAP, bool DELTA>
__global__ __launch_bounds__(ROW_THREADS, 1) void fwd_kernel(const AttnArgs a, const PlanArgs pa) {
  __shared__ __attribute__((aligned(16))) FwdShared sm;

  if (blockIdx.x == 0) {
    plan_block<ROW_THREADS>(pa, *reinterpret_cast<PlanShared*>(&sm));
    if (DELTA) {   // the full-VJP call: the dK/dV units, from the planner's ranges
      __syncthreads();
      plan_units<ROW_THREADS>(pa, a.plan.seq, *reinterpret_cast<UnitsShared*>(&sm));
    }
    return;
  }
  const int slot = (int)blockIdx.x - 1;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

  // Wave 0 finds the slot's row tile and its key steps [klo, khi) (the
  // planner's range; the other waves would only repeat its loads) and hands
  // them over through LDS.
  __shared__ int tinfo[8];
  if (wave == 0) {
    RowTile rt;
    int lo = 0, hi = 0;
    const bool ok = find_row_tile(pa, slot, rt);
    if (ok) tile_key_range(pa, rt, lo, hi);
    if (lane == 0) {
      tinfo[0] = ok ? rt.b : -1;
      tinfo[1] = rt.tile;
      tinfo[2] = rt.q0;
      tinfo[3] = rt.lq;
      tinfo[4] = rt.k0;
      tinfo[5] = rt.lk;
      tinfo[6] = lo;
      tinfo[7] = hi;
    }
  }
  __syncthreads();
  const int b = tinfo[0];
  if (b < 0) return;
  const int tile = tinfo[1];
  const int q0 = tinfo[2], Lq = tinfo[3], k0 = tinfo[4], Lk = tinfo[5];
  const int klo = tinfo[6], khi = tinfo[7];
  const int rows = Lq * a.hq;

  // copies of key step kt: waves 0-3 the K rows, waves 4-7 the V rows (one
  // 16-row group each).  Rows past Lk repeat row Lk - 1 (the tile runs before
  // the planner has cleared the zero block): only the last, masked step has
  // them, where their logits are -inf, so they add 0 * (a finite V row).
  // Issued unseen by the compiler (it would hold the step's transposing reads
  // until the next step's copies had landed); advance() orders the buffers.
  // The first step's copies go out before the Q rows are requested.
  const uint16_t* klast = a.k + (int64_t)(k0 + max(Lk, 1) - 1) * a.k_ts;
  const uint16_t* vlast = a.v + (int64_t)(k0 + max(Lk, 1) - 1) * a.v_ts;
  auto issue = [&](int kt, int buf) {
    if (wave < 4)
      load_row_tile<true>(sm.k[buf], a.k + (int64_t)k0 * a.k_ts, a.k_ts, kt * TILE_ROWS, Lk,
                          klast, wave, lane);
    else
      load_row_tile<true>(sm.v[buf], a.v + (int64_t)k0 * a.v_ts, a.v_ts, kt * TILE_ROWS, Lk,
                          vlast, wave - 4, lane);
  };
  if (klo < khi) issue(klo, klo % FWD_NBUF);

  const int row = tile * ROW_TILE + wave * 32 + l32;
  const bool row_ok = row < rows;
  const int rr = row_ok ? row : rows - 1;
  // folded row -> (token, head): R = h * Lq + i (two divisions per workgroup)
  const int hh = rr / Lq, ti = rr - hh * Lq;

  // Q row as B operand: k-step ks covers features 16ks + 8g .. +7
  const uint16_t* qrow = a.q + (int64_t)(q0 + ti) * a.q_ts + (int64_t)hh * a.q_hs + g * 8;
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = load16(qrow + ks * 16);

  const float slope2 = a.slopes[(int64_t)b * a.slopes_stride + hh] * LOG2E;
  // key j of accumulator register r in block kb of the tile at kbase is
  // kbase + 32 kb + 8 (r/4) + 4 g + r%4; cb0 - (kbase + 32 kb + 8 (r/4) + r%4)
  // is then j's signed distance from the clamped centre max(i + Lk - Lq, 0)
  const float cb0 = (float)(max(ti + Lk - Lq, 0) - 4 * g);
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)max(0, Lq - Lk - ti);
  float m = CAP ? 0.0f : -__builtin_inff();       // log2 units, relative to moff
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
  const int koff[2] = {blk_off(l32, g), blk_off(l32, 2 + g)};
  const int vi = lane & 15, vG = lane >> 4;
  const int vrow = 4 * (vG >> 1) + (vi >> 2);
  const int vcl = 2 * (vG & 1) + ((vi & 3) >> 1);
  const int voff_lo = blk_off(vrow, vcl) + 4 * (vi & 1);
  const int voff_hi = blk_off(vrow + 8, vcl) + 4 * (vi & 1);

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
  auto logits = [&](int kb, int kbase, auto masked) {
    const float cb = cb0 - (float)kbase;
    const int kleft = Lk - kbase - 4 * g;          // keys of this lane group still in range
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jl = kb * 32 + (r >> 2) * 8 + (r & 3);
      float x;
      if (CAP)
        x = __builtin_fmaf(a.lc.t_mul, cap_r(S[kb][r], a.lc),
                           -slope2 * __builtin_fabsf(cb - (float)jl));
      else
        x = __builtin_fmaf(-slope2, __builtin_fabsf(cb - (float)jl), S[kb][r] * a.lc.s_lin);
      if (decltype(masked)::value) x = jl < kleft ? x : -__builtin_inff();
      S[kb][r] = x;
    }
  };
  // P rounded to the input dtype feeds the PV product, and O is normalised by
  // the sum of those same rounded values (lsum_r), so O is an exact convex
  // combination of V rows: a single-key row reproduces v_0 and delta = dO.O
  // matches dP.  L and the backward's residual use the exact FP32 sum.
  u32x4 pb[2][2];
  auto probs = [&](int kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(S[kb][r]);
      lsum += p;
      S[kb][r] = p;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      pb[kb][s] = u32x4{pack2<T>(S[kb][8 * s + 0], S[kb][8 * s + 1]),
                        pack2<T>(S[kb][8 * s + 2], S[kb][8 * s + 3]),
                        pack2<T>(S[kb][8 * s + 4], S[kb][8 * s + 5]),
                        pack2<T>(S[kb][8 * s + 6], S[kb][8 * s + 7])};
#pragma unroll
      for (int w = 0; w < 4; ++w) lsum_r = add_pair<T>(pb[kb][s][w], lsum_r);
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

  if (CAP) {
    // The offset is fixed, so the two 32-key blocks of a step are independent.
    // Waves w and w + 4 share a SIMD; if both ran the same order they would
    // want the matrix core and the VALU at the same moments.  Wave w (lead)
    // takes a step as S0 S1 | logits/P 0 | PV0 | logits/P 1 | PV1; wave w + 4
    // (lag) defers block 1 of each step into the next one: (logits/P 1 | PV1
    // of the previous step) S0 S1 | logits/P 0 | PV0, so its VALU work falls on
    // the lead wave's products and the other way round.  A deferred block reads
    // the previous step's V tile, hence three LDS buffers.
    auto run = [&](auto lag) {
      constexpr bool LAG = decltype(lag)::value;
      auto step = [&](int kt, auto mk) {
        const int buf = kt % FWD_NBUF, kbase = kt * TILE_ROWS;
        if (LAG && kt > klo) {   // the previous step is a full one
          logits(1, kbase - TILE_ROWS, unmasked);
          probs(1);
          pv(1, sm.v[(kt - 1) % FWD_NBUF]);
        }
        scores(0, sm.k[buf]);
        scores(1, sm.k[buf]);
        logits(0, kbase, mk);
        probs(0);
        pv(0, sm.v[buf]);
        if (!LAG) {
          logits(1, kbase, mk);
          probs(1);
          pv(1, sm.v[buf]);
        }
      };
      for (int kt = klo; kt < kfull; ++kt) {
        advance(kt);
        step(kt, unmasked);
      }
      if (partial) {
        advance(nfull);
        step(nfull, masked);
      }
      if (LAG && klo < khi) {   // block 1 of the last step
        const int kt = khi - 1;
        if (partial) logits(1, kt * TILE_ROWS, masked);
        else logits(1, kt * TILE_ROWS, unmasked);
        probs(1);
        pv(1, sm.v[kt % FWD_NBUF]);
      }
    };
    if (wave < 4) run(Flag<false>{});
    else run(Flag<true>{});
  } else {
    // running maximum over both blocks of a step, then rescale
    auto step = [&](int kt, auto mk) {
      const int buf = kt % FWD_NBUF, kbase = kt * TILE_ROWS;
      scores(0, sm.k[buf]);
      scores(1, sm.k[buf]);
      logits(0, kbase, mk);
      logits(1, kbase, mk);
      float tmax = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = __builtin_fmaxf(tmax, S[kb][r]);
      tmax = __builtin_fmaxf(tmax, swap_half(tmax));
      const float mnew = __builtin_fmaxf(m, tmax);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
      lsum_r *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) O[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kb][r] -= mnew;
      probs(0);
      probs(1);
      pv(0, sm.v[buf]);
      pv(1, sm.v[buf]);
    };
    for (int kt = klo; kt < kfull; ++kt) {
      advance(kt);
      step(kt, unmasked);
    }
    if (partial) {
      advance(nfull);
      step(nfull, masked);
    }
  }

  // Epilogue.  The normalised O goes through LDS so that global stores (and
  // the dO loads of Delta) move whole 64-byte pieces of rows: in the
  // accumulator layout a lane holds 8-byte pieces of one row, which would
  // touch a new row every lane.  Delta = dO . O uses the rounded O, as the
  // standalone backward does from the stored output.
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
    eout[h] = a.out + (int64_t)(q0 + tk) * a.o_ts + (int64_t)hd * a.o_hs;
    if (DELTA) {
      const uint16_t* drow = a.dout + (int64_t)(q0 + tk) * a.do_ts + (int64_t)hd * a.do_hs;
#pragma unroll
      for (int i = 0; i < CHUNKS / 4; ++i) dpre[h][i] = load16(drow + ((lane & 3) + 4 * i) * 8);
    }
  }
  lsum += swap_half(lsum);
  lsum_r += swap_half(lsum_r);
  const float inv = lsum_r > 0.0f ? 1.0f / lsum_r : 0.0f;
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
    sinfo[lrow] = f32x4{slope2, (float)max(ti + Lk - Lq, 0), lsum > 0.0f ? -res : 0.0f, 0.0f};
    if (row_ok)
      a.lse[(int64_t)(q0 + ti) * a.hq + hh] = lsum > 0.0f ? (moff + res) * LN2 : -__builtin_inff();
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 32 + 16 * h + (lane >> 2);
    const int rg = erow[h];
    const bool ok = eok[h];
    float dpart = 0.0f;
#pragma unroll
    for (int i = 0; i < CHUNKS / 4; ++i) {
      const int c = (lane & 3) + 4 * i;
      const u32x4 o = load16(obuf + r * O_PITCH + c * 8);
      if (ok) *reinterpret_cast<u32x4*>(eout[h] + c * 8) = o;
      if (DELTA) {
        const u32x4 d = dpre[h][i];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dpart += lo_f<T>(o[e]) * lo_f<T>(d[e]) + hi_f<T>(o[e]) * hi_f<T>(d[e]);
      }
    }
    if (DELTA) {
      dpart += __shfl_xor(dpart, 1, 64);
      dpart += __shfl_xor(dpart, 2, 64);
    }
    if (ok && (lane & 3) == 0 && a.rowinfo) {
      f32x4 rec = sinfo[r];
      rec[3] = DELTA ? dpart : 0.0f;
      *reinterpret_cast<f32x4*>(a.rowinfo + ((int64_t)q0 * a.hq + rg) * 4) = rec;
    }
  }
}

template <class T>
static hipError_t launch_fwd_t(const AttnArgs& a, const PlanArgs& pa, bool cap, bool with_delta,
                               int grid, hipStream_t s) {
  if (cap) {
    if (with_delta)
      hipLaunchKernelGGL((fwd_kernel<T, true, true>), grid, ROW_THREADS, 0, s, a, pa);
    else
      hipLaunchKernelGGL((fwd_kernel<T, true, false>), grid, ROW_THREADS, 0, s, a, pa);
  } else {
    if (with_delta)
      hipLaunchKernelGGL((fwd_kernel<T, false, true>), grid, ROW_THREADS, 0, s, a, pa);
    else
      hipLaunchKernelGGL((fwd_kernel<T, false, false>), grid, ROW_THREADS, 0, s, a, pa);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, const PlanArgs& pa, int dtype, bool cap,
                      bool with_delta, hipStream_t s) {
  const int grid = 1 + a.fwd_slots;
  if (a.batch <= 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_fwd_t<BF16>(a, pa, cap, with_delta, grid, s)
                          : launch_fwd_t<F16>(a, pa, cap, with_delta, grid, s);
}

}  // namespace rga
