// Forward kernel: online-softmax attention over folded (token, head) rows.
//
// Page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section "What
// You Have": logits are (scale_multiplier / sqrt(D)) q.k, soft-capped to
// c tanh(x / c), shifted by -slope[b,h] |i + Lk - Lq - j|, then softmax-ed over
// the sequence's keys.  Page "python-20261012-ragged-flash-attention-gradient-
// recompute", section "Root causes addressed": keep a running max m and sum l
// per row, store only O and L = m + log l.
//
// Because every query head shares the one K/V head, the Lq x Hq rows of a
// sequence are folded into one M dimension (row r = token * Hq + head), so a
// workgroup's 128 rows reuse each staged K/V tile 128 times.  Each wave owns
// 32 rows and computes S^T = K Q^T (keys x rows) with Q held in registers, so
// an accumulator lane owns one row: the row max / sum need only the lane pair
// (l, l ^ 32), and O^T = V^T P^T keeps the rescale per lane.
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

template <class T, bool CAP, bool DELTA>
__global__ __launch_bounds__(WG_THREADS) void fwd_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KEY_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HEAD_DIM * LDT];

  const int rank = find_rank(a.plan.fwd_off, a.batch, blockIdx.x);
  if (rank < 0) return;
  const int b = a.plan.fwd_seq[rank];
  const int tile = blockIdx.x - a.plan.fwd_off[rank];
  const int* sq = a.plan.seq + b * SEQ_FIELDS;
  const int q0 = sq[SQ_Q0], Lq = sq[SQ_LQ], k0 = sq[SQ_K0], Lk = sq[SQ_LK];
  const int rows = sq[SQ_ROWS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int row = tile * ROW_TILE + wave * 32 + l32;
  const bool row_ok = row < rows;
  const int rr = row_ok ? row : rows - 1;
  const int ti = rr / a.hq;
  const int hh = rr - ti * a.hq;

  // Q row as B operand: k-step ks covers features 16ks + 8g .. +7.
  const uint16_t* qrow = a.q + (int64_t)(q0 + ti) * a.q_ts + (int64_t)hh * a.q_hs;
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = load16(qrow + ks * 16 + g * 8);

  const float slope2 = a.slopes[(int64_t)b * a.slopes_stride + hh] * LOG2E;
  // distance of key j is |cpos - j|; this lane's keys in block kb are
  // kbase + 32 kb + 8 (r/4) + 4 g + r%4.
  const float cpos = (float)(ti + Lk - Lq) - (float)(4 * g);

  float m = -__builtin_inff();
  float lsum = 0.0f;
  f32x16 O[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) O[db] = f32x16{};

  const int ntiles = (Lk + KEY_STEP - 1) / KEY_STEP;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int kbase = kt * KEY_STEP;
    __syncthreads();
    stage_keys_rowmajor(Ks, a.k, a.k_ts, k0, Lk, kbase);
    stage_keys_transposed<false>(Vt, nullptr, a.v, a.v_ts, k0, Lk, kbase);
    __syncthreads();

    f32x16 S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = f32x16{};
      const uint16_t* kp = Ks + (kb * 32 + l32) * LDK + g * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        S[kb] = mfma32<T>(load16(kp + ks * 16), qf[ks], S[kb]);
    }

    // logits, masked past the sequence end
    float tmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = kb * 32 + (r >> 2) * 8 + (r & 3);       // key offset without 4g
        float rc;
        float x = logit2<CAP>(S[kb][r], slope2, cpos - (float)(kbase + jl), a.lc, rc);
        x = (kbase + jl + 4 * g < Lk) ? x : -__builtin_inff();
        S[kb][r] = x;
        tmax = __builtin_fmaxf(tmax, x);
      }
    }
    tmax = __builtin_fmaxf(tmax, swap_half(tmax));
    const float mnew = __builtin_fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;

    float psum = 0.0f;
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(S[kb][r] - mnew);
        psum += p;
        S[kb][r] = p;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pb[kb][s] = u32x4{pack2<T>(S[kb][8 * s + 0], S[kb][8 * s + 1]),
                          pack2<T>(S[kb][8 * s + 2], S[kb][8 * s + 3]),
                          pack2<T>(S[kb][8 * s + 4], S[kb][8 * s + 5]),
                          pack2<T>(S[kb][8 * s + 6], S[kb][8 * s + 7])};
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) O[db] *= alpha;

    // O^T[d][row] += V^T[d][keys] P^T[keys][row]
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const uint16_t* vp = Vt + (db * 32 + l32) * LDT + g * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          O[db] = mfma32<T>(read_perm_a(vp + kb * 32 + s * 16), pb[kb][s], O[db]);
    }
  }

  // epilogue: normalise, store O (feature 32db + 8(r/4) + 4g + r%4), L, and delta
  lsum += swap_half(lsum);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  uint16_t* orow = a.out + (int64_t)(q0 + ti) * a.o_ts + (int64_t)hh * a.o_hs + g * 4;
  const uint16_t* dorow = nullptr;
  if (DELTA) dorow = a.dout + (int64_t)(q0 + ti) * a.do_ts + (int64_t)hh * a.do_hs + g * 4;
  float dsum = 0.0f;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const float o0 = O[db][rq * 4 + 0] * inv, o1 = O[db][rq * 4 + 1] * inv;
      const float o2 = O[db][rq * 4 + 2] * inv, o3 = O[db][rq * 4 + 3] * inv;
      const int off = db * 32 + rq * 8;
      if (row_ok)
        *reinterpret_cast<u32x2*>(orow + off) = u32x2{pack2<T>(o0, o1), pack2<T>(o2, o3)};
      if (DELTA) {
        const u32x2 d = *reinterpret_cast<const u32x2*>(dorow + off);
        dsum += o0 * lo_f<T>(d[0]) + o1 * hi_f<T>(d[0]) + o2 * lo_f<T>(d[1]) + o3 * hi_f<T>(d[1]);
      }
    }
  }
  if (DELTA) dsum += swap_half(dsum);
  if (row_ok && g == 0) {
    const int64_t ri = (int64_t)(q0 + ti) * a.hq + hh;
    a.lse[ri] = lsum > 0.0f ? (m + fast_log2(lsum)) * LN2 : -__builtin_inff();
    if (DELTA) a.delta[ri] = dsum;
  }
}

template <class T>
static hipError_t launch_fwd_t(const AttnArgs& a, bool cap, bool with_delta, int grid,
                               hipStream_t s) {
  if (cap) {
    if (with_delta) hipLaunchKernelGGL((fwd_kernel<T, true, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<T, true, false>), grid, WG_THREADS, 0, s, a);
  } else {
    if (with_delta) hipLaunchKernelGGL((fwd_kernel<T, false, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<T, false, false>), grid, WG_THREADS, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, int dtype, bool cap, bool with_delta, int grid,
                      hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_fwd_t<BF16>(a, cap, with_delta, grid, s)
                          : launch_fwd_t<F16>(a, cap, with_delta, grid, s);
}

}  // namespace rga
