// Backward kernels: recompute P from the stored row statistic L, then
//   dP = dO V^T,  dS = P * (dP - Delta) * (1 - tanh^2(s / c)),
//   dQ = sigma dS K,  dK = sigma sum_rows dS^T Q,  dV = sum_rows P^T dO.
//
// Page "python-20261012-ragged-flash-attention-gradient-recompute", section
// "Root causes addressed": no probability matrix is stored; the backward
// rebuilds each tile from L.  Page "Noncausal Global Extreme-GQA Ragged
// Attention Full VJP", section "Hard Constraints": the K/V gradients reduce over
// every query head sharing the K/V head, and the cap sits between the scaled
// dot product and ALiBi, so its derivative multiplies dP - Delta.
//
// With r = 1 / (1 + e^{2s/c}), 1 - tanh^2(s/c) = 4 r (1 - r); the kernels form
// r - r^2 and fold the factor 4 into the final sigma scale of dQ and dK.
//
// P is rebuilt exactly as the forward formed it: distances from the clamped
// centre max(i + Lk - Lq, 0), the large per-row offset kept analytic, and only
// the small residual log2 l subtracted (see fwd.hip), so no two large numbers
// are ever subtracted.
//
// dK/dV: a workgroup owns 128 keys of one sequence (4 waves x 32 keys, K and V
// in registers) and walks a chunk of that sequence's folded (token, head) rows
// 32 at a time, so the sum over all Hq heads happens in registers in a fixed
// order.  Sequences split into several row chunks write FP32 partials that a
// separate pass adds in chunk order; no atomics anywhere.
//
// dQ: a workgroup owns 256 folded rows (like the forward) and walks the keys.
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

// Residual log2 l of row ri relative to its offset m_i, from the forward's
// residual array or, for a stored natural-log L, as L log2(e) - m_i.
template <bool CAP>
__device__ __forceinline__ float row_residual(const AttnArgs& a, int64_t ri, float slope2,
                                              int dmin) {
  if (a.lres) return a.lres[ri];
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)dmin;
  return a.lse[ri] * LOG2E - moff;
}

template <class T, bool CAP>
__global__ __launch_bounds__(KV_THREADS, 1) void dkdv_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][KV_ROW_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[2][KV_ROW_STEP * LDK];
  // per row: slope * log2(e), clamped ALiBi centre, -residual, delta
  __shared__ __attribute__((aligned(16))) f32x4 rinfo[2][KV_ROW_STEP];

  const int rank = find_rank(a.plan.kv_off, a.batch, blockIdx.x);
  if (rank < 0) return;
  const int b = a.plan.kv_seq[rank];
  const int unit = blockIdx.x - a.plan.kv_off[rank];
  const int* sq = a.plan.seq + b * SEQ_FIELDS;
  const int q0 = sq[SQ_Q0], Lq = sq[SQ_LQ], k0 = sq[SQ_K0], Lk = sq[SQ_LK];
  const int rows = sq[SQ_ROWS], nchunk = sq[SQ_NCHUNK], chunk = sq[SQ_CHUNK];
  const int ktile = unit / nchunk;
  const int ci = unit - ktile * nchunk;
  const int row_begin = ci * chunk;
  const int row_end = min(rows, row_begin + chunk);
  const int hq = a.hq;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wkey0 = ktile * KEY_TILE + wave * 32;   // first key of this wave
  const bool wave_active = wkey0 < Lk;
  const int key = wkey0 + l32;
  const bool key_ok = key < Lk;
  const int kk = key_ok ? key : Lk - 1;

  // K and V rows as B operands (lane = key)
  u32x4 kf[KSTEPS], vf[KSTEPS];
  {
    const uint16_t* kr = a.k + (int64_t)(k0 + kk) * a.k_ts + g * 8;
    const uint16_t* vr = a.v + (int64_t)(k0 + kk) * a.v_ts + g * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kf[ks] = key_ok ? load16(kr + ks * 16) : u32x4{0u, 0u, 0u, 0u};
      vf[ks] = key_ok ? load16(vr + ks * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float keyf = (float)key;

  // per-row facts of rows [r0, r0 + 32), computed by threads 0..31
  auto row_info = [&](int r0) {
    const int r = r0 + tid;
    f32x4 info = {0.0f, 0.0f, -__builtin_inff(), 0.0f};   // padding row: P = 0
    if (r < row_end) {
      const int t0 = r / hq, h0 = r - t0 * hq;
      const int64_t ri = (int64_t)(q0 + t0) * hq + h0;
      const float slope2 = a.slopes[(int64_t)b * a.slopes_stride + h0] * LOG2E;
      info[0] = slope2;
      info[1] = (float)max(t0 + Lk - Lq, 0);
      info[2] = -row_residual<CAP>(a, ri, slope2, max(0, Lq - Lk - t0));
      info[3] = a.delta[ri];
    }
    return info;
  };

  f32x16 dK[DBLK], dV[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) { dK[db] = f32x16{}; dV[db] = f32x16{}; }

  PairStager<KV_THREADS, KV_ROW_STEP> st;
  f32x4 info_next = {0.0f, 0.0f, 0.0f, 0.0f};
  if (row_begin < row_end) {
    st.load_rows(a.q, a.q_ts, a.q_hs, a.dout, a.do_ts, a.do_hs, q0, hq, row_begin, row_end);
    st.template store<LDK, LDK>(Qs[0], Ds[0]);
    if (tid < KV_ROW_STEP) rinfo[0][tid] = row_info(row_begin);
  }
  __syncthreads();

  int buf = 0;
  for (int r0 = row_begin; r0 < row_end; r0 += KV_ROW_STEP, buf ^= 1) {
    const bool more = r0 + KV_ROW_STEP < row_end;
    if (more) {
      st.load_rows(a.q, a.q_ts, a.q_hs, a.dout, a.do_ts, a.do_hs, q0, hq, r0 + KV_ROW_STEP,
                   row_end);
      if (tid < KV_ROW_STEP) info_next = row_info(r0 + KV_ROW_STEP);
    }
    if (wave_active) {
      const uint16_t* Qb = Qs[buf];
      const uint16_t* Db = Ds[buf];
      // S[row][key], dP[row][key]: A = Q / dO rows from LDS, B = K / V registers
      f32x16 S = f32x16{}, dP = f32x16{};
      {
        const uint16_t* qp = Qb + l32 * LDK + g * 8;
        const uint16_t* dp = Db + l32 * LDK + g * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          S = mfma32<T>(load16(qp + ks * 16), kf[ks], S);
          dP = mfma32<T>(load16(dp + ks * 16), vf[ks], dP);
        }
      }
      // rows owned by this lane: 8 (r/4) + 4 g + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const f32x4 ri = rinfo[buf][(r >> 2) * 8 + g * 4 + (r & 3)];
        const float bias = __builtin_fmaf(-ri[0], __builtin_fabsf(ri[1] - keyf), ri[2]);
        float p, w;
        if (CAP) {
          const float rc = cap_r(S[r], a.lc);
          p = fast_exp2(__builtin_fmaf(a.lc.t_mul, rc, bias));
          w = __builtin_fmaf(-rc, rc, rc);
        } else {
          p = fast_exp2(__builtin_fmaf(S[r], a.lc.s_lin, bias));
          w = 1.0f;
        }
        S[r] = p;
        dP[r] = p * (dP[r] - ri[3]) * w;
      }
      u32x4 pb[2], sb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        pb[s] = u32x4{pack2<T>(S[8 * s + 0], S[8 * s + 1]), pack2<T>(S[8 * s + 2], S[8 * s + 3]),
                      pack2<T>(S[8 * s + 4], S[8 * s + 5]), pack2<T>(S[8 * s + 6], S[8 * s + 7])};
        sb[s] = u32x4{pack2<T>(dP[8 * s + 0], dP[8 * s + 1]), pack2<T>(dP[8 * s + 2], dP[8 * s + 3]),
                      pack2<T>(dP[8 * s + 4], dP[8 * s + 5]), pack2<T>(dP[8 * s + 6], dP[8 * s + 7])};
      }
      // dV^T[d][key] += dO^T[d][rows] P[rows][key];  dK^T likewise with Q^T and dS
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          dV[db] = mfma32<T>(read_tr_a<LDK>(Db, s * 16, db * 32, lane), pb[s], dV[db]);
          dK[db] = mfma32<T>(read_tr_a<LDK>(Qb, s * 16, db * 32, lane), sb[s], dK[db]);
        }
    }
    if (more) {
      st.template store<LDK, LDK>(Qs[buf ^ 1], Ds[buf ^ 1]);
      if (tid < KV_ROW_STEP) rinfo[buf ^ 1][tid] = info_next;
    }
    __syncthreads();
  }

  if (!key_ok) return;
  // lane owns key `key`, features 32db + 8(r/4) + 4g + r%4
  const float ks_scale = CAP ? 4.0f * a.lc.sigma : a.lc.sigma;
  if (nchunk == 1) {
    uint16_t* dkr = a.dk + (int64_t)(k0 + key) * a.dk_ts + g * 4;
    uint16_t* dvr = a.dv + (int64_t)(k0 + key) * a.dv_ts + g * 4;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int off = db * 32 + rq * 8;
        const f32x16& K = dK[db];
        const f32x16& V = dV[db];
        *reinterpret_cast<u32x2*>(dkr + off) =
            u32x2{pack2<T>(ks_scale * K[rq * 4 + 0], ks_scale * K[rq * 4 + 1]),
                  pack2<T>(ks_scale * K[rq * 4 + 2], ks_scale * K[rq * 4 + 3])};
        *reinterpret_cast<u32x2*>(dvr + off) =
            u32x2{pack2<T>(V[rq * 4 + 0], V[rq * 4 + 1]), pack2<T>(V[rq * 4 + 2], V[rq * 4 + 3])};
      }
  } else {
    const int64_t slot = (int64_t)blockIdx.x * KEY_TILE + wave * 32 + l32;
    float* pk = a.part_dk + slot * HEAD_DIM + g * 4;
    float* pv = a.part_dv + slot * HEAD_DIM + g * 4;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int off = db * 32 + rq * 8;
        *reinterpret_cast<f32x4*>(pk + off) =
            f32x4{ks_scale * dK[db][rq * 4 + 0], ks_scale * dK[db][rq * 4 + 1],
                  ks_scale * dK[db][rq * 4 + 2], ks_scale * dK[db][rq * 4 + 3]};
        *reinterpret_cast<f32x4*>(pv + off) =
            f32x4{dV[db][rq * 4 + 0], dV[db][rq * 4 + 1], dV[db][rq * 4 + 2], dV[db][rq * 4 + 3]};
      }
  }
}

template <class T, bool CAP>
__global__ __launch_bounds__(ROW_THREADS, 1) void dq_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KEY_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KEY_STEP * LDK];

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
  const int64_t ri = (int64_t)(q0 + ti) * a.hq + hh;

  const uint16_t* qrow = a.q + (int64_t)(q0 + ti) * a.q_ts + (int64_t)hh * a.q_hs + g * 8;
  const uint16_t* dorow = a.dout + (int64_t)(q0 + ti) * a.do_ts + (int64_t)hh * a.do_hs + g * 8;
  u32x4 qf[KSTEPS], df[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = load16(qrow + ks * 16);
    df[ks] = load16(dorow + ks * 16);
  }
  const float slope2 = a.slopes[(int64_t)b * a.slopes_stride + hh] * LOG2E;
  const float cb0 = (float)(max(ti + Lk - Lq, 0) - 4 * g);
  const float boff = Lk > 0 ? -row_residual<CAP>(a, ri, slope2, max(0, Lq - Lk - ti)) : 0.0f;
  const float dl = Lk > 0 ? a.delta[ri] : 0.0f;

  f32x16 dQ[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dQ[db] = f32x16{};

  const int ntiles = (Lk + KEY_STEP - 1) / KEY_STEP;
  PairStager<ROW_THREADS, KEY_STEP> st;
  if (ntiles > 0) {
    st.load_keys(a.k, a.k_ts, a.v, a.v_ts, k0, min(Lk, KEY_STEP));
    st.template store<LDK, LDK>(Ks[0], Vs[0]);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int kbase = kt * KEY_STEP;
    const bool more = kt + 1 < ntiles;
    if (more)
      st.load_keys(a.k, a.k_ts, a.v, a.v_ts, (int64_t)k0 + kbase + KEY_STEP,
                   Lk - kbase - KEY_STEP);
    const uint16_t* Kb = Ks[kt & 1];
    const uint16_t* Vb = Vs[kt & 1];
    const float cb = cb0 - (float)kbase;
    const bool full = kbase + KEY_STEP <= Lk;
    const int kleft = Lk - kbase - 4 * g;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T[key][row] = K Q^T and dP^T[key][row] = V dO^T (lane = row)
      f32x16 S = f32x16{}, dP = f32x16{};
      const uint16_t* kp = Kb + (kb * 32 + l32) * LDK + g * 8;
      const uint16_t* vp = Vb + (kb * 32 + l32) * LDK + g * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        S = mfma32<T>(load16(kp + ks * 16), qf[ks], S);
        dP = mfma32<T>(load16(vp + ks * 16), df[ks], dP);
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
        if (!full) p = jl < kleft ? p : 0.0f;
        S[r] = p * (dP[r] - dl) * w;
      }
      u32x4 sb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        sb[s] = u32x4{pack2<T>(S[8 * s + 0], S[8 * s + 1]), pack2<T>(S[8 * s + 2], S[8 * s + 3]),
                      pack2<T>(S[8 * s + 4], S[8 * s + 5]), pack2<T>(S[8 * s + 6], S[8 * s + 7])};
      // dQ^T[d][row] += K^T[d][keys] dS^T[keys][row]
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          dQ[db] = mfma32<T>(read_tr_a<LDK>(Kb, kb * 32 + s * 16, db * 32, lane), sb[s], dQ[db]);
    }
    if (more) st.template store<LDK, LDK>(Ks[(kt + 1) & 1], Vs[(kt + 1) & 1]);
    __syncthreads();
  }

  if (!row_ok) return;
  const float scale = CAP ? 4.0f * a.lc.sigma : a.lc.sigma;
  uint16_t* dqr = a.dq + (int64_t)(q0 + ti) * a.dq_ts + (int64_t)hh * a.dq_hs + g * 4;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *reinterpret_cast<u32x2*>(dqr + db * 32 + rq * 8) =
          u32x2{pack2<T>(scale * dQ[db][rq * 4 + 0], scale * dQ[db][rq * 4 + 1]),
                pack2<T>(scale * dQ[db][rq * 4 + 2], scale * dQ[db][rq * 4 + 3])};
}

template <class T>
static hipError_t launch_dkdv_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  if (cap) hipLaunchKernelGGL((dkdv_kernel<T, true>), grid, KV_THREADS, 0, s, a);
  else hipLaunchKernelGGL((dkdv_kernel<T, false>), grid, KV_THREADS, 0, s, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_dq_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  if (cap) hipLaunchKernelGGL((dq_kernel<T, true>), grid, ROW_THREADS, 0, s, a);
  else hipLaunchKernelGGL((dq_kernel<T, false>), grid, ROW_THREADS, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dkdv(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_dkdv_t<BF16>(a, cap, grid, s)
                          : launch_dkdv_t<F16>(a, cap, grid, s);
}

hipError_t launch_dq(const AttnArgs& a, int dtype, bool cap, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_dq_t<BF16>(a, cap, grid, s)
                          : launch_dq_t<F16>(a, cap, grid, s);
}

}  // namespace rga
