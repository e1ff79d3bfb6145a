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
// dK/dV: a workgroup owns 128 keys of one sequence (4 waves x 32 keys, K and V
// in registers) and walks a chunk of that sequence's folded (token, head) rows
// 32 at a time, so the sum over all Hq heads happens in registers in a fixed
// order.  Sequences split into several row chunks write FP32 partials that a
// separate pass adds in chunk order; no atomics anywhere.
//
// dQ: a workgroup owns 128 folded rows (like the forward) and walks the keys.
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

// Row tiles of the dK/dV kernel: row-major [32][LDK] and transposed [160][LDR].
// LDR = 36 halves (18 dwords) keeps 8-byte reads of 16 consecutive feature rows
// conflict-free.
constexpr int LDR = KV_ROW_STEP + 4;

template <class T, bool CAP>
__global__ __launch_bounds__(WG_THREADS) void dkdv_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[KV_ROW_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[KV_ROW_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[HEAD_DIM * LDR];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[HEAD_DIM * LDR];
  __shared__ __attribute__((aligned(16))) f32x4 rinfo[KV_ROW_STEP];  // slope2, cpos, L2, delta

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

  // K and V rows as B operands (lane = key).
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

  f32x16 dK[DBLK], dV[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) { dK[db] = f32x16{}; dV[db] = f32x16{}; }

  for (int r0 = row_begin; r0 < row_end; r0 += KV_ROW_STEP) {
    __syncthreads();
    // stage 32 rows of Q and dO in both layouts; task = row pair x 16-byte chunk
    for (int t = tid; t < 2 * (KV_ROW_STEP / 2) * CHUNKS; t += WG_THREADS) {
      const int which = t / ((KV_ROW_STEP / 2) * CHUNKS);
      const int u = t - which * ((KV_ROW_STEP / 2) * CHUNKS);
      const int rp = u % (KV_ROW_STEP / 2);
      const int c = u / (KV_ROW_STEP / 2);
      const int lr = 2 * rp;
      const uint16_t* base = which ? a.dout : a.q;
      const int64_t ts = which ? a.do_ts : a.q_ts;
      const int64_t hs = which ? a.do_hs : a.q_hs;
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
      const int ra = r0 + lr, rb = r0 + lr + 1;
      if (ra < row_end) {
        const int t0 = ra / hq, h0 = ra - t0 * hq;
        x0 = load16(base + (int64_t)(q0 + t0) * ts + (int64_t)h0 * hs + c * 8);
      }
      if (rb < row_end) {
        const int t1 = rb / hq, h1 = rb - t1 * hq;
        x1 = load16(base + (int64_t)(q0 + t1) * ts + (int64_t)h1 * hs + c * 8);
      }
      uint16_t* rm = which ? Ds : Qs;
      uint16_t* tr = which ? Dt : Qt;
      *reinterpret_cast<u32x4*>(rm + lr * LDK + c * 8) = x0;
      *reinterpret_cast<u32x4*>(rm + (lr + 1) * LDK + c * 8) = x1;
      uint16_t* col = tr + (c * 8) * LDR + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t*>(col + (2 * e) * LDR) = interleave_lo(x0[e], x1[e]);
        *reinterpret_cast<uint32_t*>(col + (2 * e + 1) * LDR) = interleave_hi(x0[e], x1[e]);
      }
    }
    if (tid < KV_ROW_STEP) {
      const int r = r0 + tid;
      f32x4 info = {0.0f, 0.0f, __builtin_inff(), 0.0f};   // padding row: P = 0
      if (r < row_end) {
        const int t0 = r / hq, h0 = r - t0 * hq;
        const int64_t ri = (int64_t)(q0 + t0) * hq + h0;
        info[0] = a.slopes[(int64_t)b * a.slopes_stride + h0] * LOG2E;
        info[1] = (float)(t0 + Lk - Lq);
        info[2] = a.lse[ri] * LOG2E;
        info[3] = a.delta[ri];
      }
      rinfo[tid] = info;
    }
    __syncthreads();
    if (!wave_active) continue;

    // S[row][key] and dP[row][key]: A = Q / dO rows from LDS, B = K / V registers
    f32x16 S = f32x16{}, dP = f32x16{};
    {
      const uint16_t* qp = Qs + l32 * LDK + g * 8;
      const uint16_t* dp = Ds + l32 * LDK + g * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        S = mfma32<T>(load16(qp + ks * 16), kf[ks], S);
        dP = mfma32<T>(load16(dp + ks * 16), vf[ks], dP);
      }
    }
    // rows owned by this lane: 8 (r/4) + 4 g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const f32x4 ri = rinfo[(r >> 2) * 8 + g * 4 + (r & 3)];
      float rc;
      const float x = logit2<CAP>(S[r], ri[0], ri[1] - keyf, a.lc, rc);
      const float p = fast_exp2(x - ri[2]);
      float ds = p * (dP[r] - ri[3]);
      if (CAP) ds *= 4.0f * rc * (1.0f - rc);
      S[r] = p;
      dP[r] = ds;
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
    for (int db = 0; db < DBLK; ++db) {
      const uint16_t* dtp = Dt + (db * 32 + l32) * LDR + g * 4;
      const uint16_t* qtp = Qt + (db * 32 + l32) * LDR + g * 4;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        dV[db] = mfma32<T>(read_perm_a(dtp + s * 16), pb[s], dV[db]);
        dK[db] = mfma32<T>(read_perm_a(qtp + s * 16), sb[s], dK[db]);
      }
    }
  }

  if (!key_ok) return;
  // lane owns key `key`, features 32db + 8(r/4) + 4g + r%4
  const float sigma = a.lc.sigma;
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
            u32x2{pack2<T>(sigma * K[rq * 4 + 0], sigma * K[rq * 4 + 1]),
                  pack2<T>(sigma * K[rq * 4 + 2], sigma * K[rq * 4 + 3])};
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
            f32x4{sigma * dK[db][rq * 4 + 0], sigma * dK[db][rq * 4 + 1],
                  sigma * dK[db][rq * 4 + 2], sigma * dK[db][rq * 4 + 3]};
        *reinterpret_cast<f32x4*>(pv + off) =
            f32x4{dV[db][rq * 4 + 0], dV[db][rq * 4 + 1], dV[db][rq * 4 + 2], dV[db][rq * 4 + 3]};
      }
  }
}

template <class T, bool CAP>
__global__ __launch_bounds__(WG_THREADS) void dq_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KEY_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KEY_STEP * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[HEAD_DIM * LDT];

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
  const float cpos = (float)(ti + Lk - Lq) - (float)(4 * g);
  const float L2 = Lk > 0 ? a.lse[ri] * LOG2E : 0.0f;
  const float dl = Lk > 0 ? a.delta[ri] : 0.0f;

  f32x16 dQ[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dQ[db] = f32x16{};

  const int ntiles = (Lk + KEY_STEP - 1) / KEY_STEP;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int kbase = kt * KEY_STEP;
    __syncthreads();
    stage_keys_transposed<true>(Kt, Ks, a.k, a.k_ts, k0, Lk, kbase);
    stage_keys_rowmajor(Vs, a.v, a.v_ts, k0, Lk, kbase);
    __syncthreads();

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T[key][row] = K Q^T and dP^T[key][row] = V dO^T (lane = row)
      f32x16 S = f32x16{}, dP = f32x16{};
      const uint16_t* kp = Ks + (kb * 32 + l32) * LDK + g * 8;
      const uint16_t* vp = Vs + (kb * 32 + l32) * LDK + g * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        S = mfma32<T>(load16(kp + ks * 16), qf[ks], S);
        dP = mfma32<T>(load16(vp + ks * 16), df[ks], dP);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = kbase + kb * 32 + (r >> 2) * 8 + (r & 3);
        float rc;
        const float x = logit2<CAP>(S[r], slope2, cpos - (float)jl, a.lc, rc);
        float p = fast_exp2(x - L2);
        p = (jl + 4 * g < Lk) ? p : 0.0f;
        float ds = p * (dP[r] - dl);
        if (CAP) ds *= 4.0f * rc * (1.0f - rc);
        S[r] = ds;
      }
      u32x4 sb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        sb[s] = u32x4{pack2<T>(S[8 * s + 0], S[8 * s + 1]), pack2<T>(S[8 * s + 2], S[8 * s + 3]),
                      pack2<T>(S[8 * s + 4], S[8 * s + 5]), pack2<T>(S[8 * s + 6], S[8 * s + 7])};
      // dQ^T[d][row] += K^T[d][keys] dS^T[keys][row]
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const uint16_t* ktp = Kt + (db * 32 + l32) * LDT + kb * 32 + g * 4;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          dQ[db] = mfma32<T>(read_perm_a(ktp + s * 16), sb[s], dQ[db]);
      }
    }
  }

  if (!row_ok) return;
  const float sigma = a.lc.sigma;
  uint16_t* dqr = a.dq + (int64_t)(q0 + ti) * a.dq_ts + (int64_t)hh * a.dq_hs + g * 4;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *reinterpret_cast<u32x2*>(dqr + db * 32 + rq * 8) =
          u32x2{pack2<T>(sigma * dQ[db][rq * 4 + 0], sigma * dQ[db][rq * 4 + 1]),
                pack2<T>(sigma * dQ[db][rq * 4 + 2], sigma * dQ[db][rq * 4 + 3])};
}

template <class T>
static hipError_t launch_dkdv_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  if (cap) hipLaunchKernelGGL((dkdv_kernel<T, true>), grid, WG_THREADS, 0, s, a);
  else hipLaunchKernelGGL((dkdv_kernel<T, false>), grid, WG_THREADS, 0, s, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_dq_t(const AttnArgs& a, bool cap, int grid, hipStream_t s) {
  if (cap) hipLaunchKernelGGL((dq_kernel<T, true>), grid, WG_THREADS, 0, s, a);
  else hipLaunchKernelGGL((dq_kernel<T, false>), grid, WG_THREADS, 0, s, a);
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
