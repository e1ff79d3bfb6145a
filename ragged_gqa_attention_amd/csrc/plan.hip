// Device planner, fixed-order K/V partial reduction, and the backward's row
// records for the standalone backward entry.
//
// The planner reads cu_q / cu_k on the device (no host synchronisation) and
// builds two work lists for the packed ragged batch (page "Noncausal Global
// Extreme-GQA Ragged Attention Full VJP", section "What You Have": 18-52
// sequences whose Q/K length ratio runs both ways):
//   * row tiles (forward, dQ): ceil(Lq * Hq / 256) per sequence, sequences
//     ranked by Lk, largest first, so the longest work starts first;
//   * dK/dV units: each 128-key tile of a sequence splits the row tiles that
//     visit it (whose key-step range meets it, see row_key_steps) into runs of
//     near-equal length, sized so that the units fill whole rounds of the
//     compute units.
// Each workgroup finds its item in a map with one load.
#include "dropout.hpp"
#include "kernels.hpp"
#include "planner.hpp"
#include "tiles.hpp"

namespace rga {

constexpr int PLAN_THREADS = 256;
constexpr int WG_THREADS = 256;          // row-record kernel


// The planner alone (the standalone backward entry and an empty batch; the
// forward's grid holds it otherwise).
__global__ __launch_bounds__(PLAN_THREADS) void prep_kernel(const PlanArgs pa) {
  __shared__ __attribute__((aligned(16))) PlanShared sm;
  plan_block<PLAN_THREADS>(pa, sm);
}

hipError_t launch_prep(const PlanArgs& pa, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, 1, PLAN_THREADS, 0, s, pa);
  return hipGetLastError();
}

// Row records for the backward entry that starts from a saved forward:
// Delta = sum_d dout[row, d] * out[row, d] over the stored 16-bit output, the
// slope in base-2 units, the ALiBi centre (clamped at 0 unless a window or
// causal mask is set, whose test needs the unclamped one) and the base-2 residual of
// the stored natural-log L relative to the row offset the forward used (see
// fwd.hip).  Eight lanes share a row; each reads 16-byte chunks.
template <class T, int D, bool CAP>
__global__ __launch_bounds__(WG_THREADS) void rowinfo_kernel(const AttnArgs a) {
  constexpr int CHUNKS = Geo<D>::CHUNKS;
  const int64_t gid = (int64_t)blockIdx.x * WG_THREADS + threadIdx.x;
  const int64_t r = gid >> 3;
  const int sub = (int)(gid & 7);
  const int64_t nrows = a.total_q * a.hq;
  const bool ok = r < nrows;
  const int64_t t = ok ? r / a.hq : 0;
  const int h = (int)(r - t * a.hq);
  float acc = 0.0f;
  if (ok) {
    const uint16_t* o = a.out + t * a.o_ts + (int64_t)h * a.o_hs;
    const uint16_t* d = a.dout + t * a.do_ts + (int64_t)h * a.do_hs;
    for (int c = sub; c < CHUNKS; c += 8) {
      const u32x4 x = load16(o + c * 8), y = load16(d + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc += lo_f<T>(x[e]) * lo_f<T>(y[e]) + hi_f<T>(x[e]) * hi_f<T>(y[e]);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (!ok || sub != 0) return;
  // packed sequence of token t: the last b with q0(b) <= t (never an empty
  // one), searched over the plan records of its first K/V head (v = b hkv)
  const int* seq = a.plan.seq;
  const int nb = a.batch / a.hkv;
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq[mid * a.hkv * SEQ_FIELDS + SQ_Q0] <= t) lo = mid; else hi = mid - 1;
  }
  const int* s = seq + lo * a.hkv * SEQ_FIELDS;
  const int i = (int)(t - s[SQ_Q0]);
  const int Lq = s[SQ_LQ], Lk = s[SQ_LK];
  // folded row record: head-major over the packed sequence's hq heads, so the
  // rows of the group of K/V head g start at q0 hq + g group Lq
  const int64_t fr = (int64_t)s[SQ_Q0] * a.hq + (int64_t)h * Lq + i;
  const float slope2 = a.slopes[(int64_t)lo * a.slopes_stride + h] * LOG2E;
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)max(0, Lq - Lk - i);
  const float L = a.lse[r];
  const float negres = Lk > 0 ? moff - L * LOG2E : 0.0f;
  const bool win = a.win_left >= 0 || a.win_right >= 0;
  *reinterpret_cast<f32x4*>(a.rowinfo + fr * 4) =
      f32x4{slope2, (float)(win ? i + Lk - Lq : max(i + Lk - Lq, 0)), negres, acc};
  if (a.drop_on) a.droprec[fr] = drop_row(a, lo, h, i, t);
}

// Key-step ranges of the standalone backward (the full-VJP call takes the
// forward's): one workgroup per 256-row tile, a thread per row, from the row
// records.  The row's bound is SKIP_UNDERFLOW plus its own residual (the
// residual comes from the caller's L, so it is not bounded by the cap); a
// row whose residual is not finite keeps every key.
__global__ __launch_bounds__(WG_THREADS) void ksteps_kernel(const AttnArgs a) {
  static_assert(WG_THREADS == ROW_TILE, "a thread per row of the tile");
  __shared__ int span[2][WG_THREADS / 64];
  const int b = a.plan.fwd_map[2 * blockIdx.x];
  if (b < 0) return;
  const int tile = a.plan.fwd_map[2 * blockIdx.x + 1];
  const int* sq = a.plan.seq + b * SEQ_FIELDS;
  const int R = tile * ROW_TILE + (int)threadIdx.x;
  const bool ok = R < sq[SQ_ROWS];
  const int Lk = sq[SQ_LK];
  float slope2 = 0.0f, thr = 0.0f;
  int centre = 0;
  if (ok && Lk > 0) {
    const f32x4 info = *reinterpret_cast<const f32x4*>(
        a.rowinfo + ((int64_t)sq[SQ_Q0] * a.hq + (int64_t)sq[SQ_HB] * sq[SQ_LQ] + R) * 4);
    slope2 = info[0];
    centre = max((int)info[1], 0);   // unclamped under a window
    const float radd = info[2];   // added to every exponent of the row
    if (a.skip_log2 > 0.0f && __builtin_isfinite(radd))
      thr = SKIP_UNDERFLOW + __builtin_fmaxf(radd, 0.0f);
  }
  int lo, hi;
  row_key_steps(ok, slope2, centre, Lk, thr, lo, hi);
  if (ok && Lk > 0 && (a.win_left >= 0 || a.win_right >= 0)) {
    // only the steps that hold the row's window keys
    int i, h;
    unfold_row(R, sq, i, h);
    int wlo, whi;
    token_range_steps(i, i, sq[SQ_LQ], Lk, -1, a.win_left, a.win_right, wlo, whi);
    lo = max(lo, wlo);
    hi = min(hi, whi);
    if (lo >= hi) {
      lo = 0x7fffffff;
      hi = 0;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  if (lane == 0) {
    span[0][wave] = lo;
    span[1][wave] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < WG_THREADS / 64; ++w) {
      lo = min(lo, span[0][w]);
      hi = max(hi, span[1][w]);
    }
    finish_range(lo, hi);
    int* ks = a.ksteps + 2 * (sq[SQ_RTOFF] + tile);
    ks[0] = lo;
    ks[1] = hi;
  }
}

// dK/dV units of the standalone backward, planned after ksteps_kernel has
// written the ranges (one workgroup; the sequence records are in global memory).
__global__ __launch_bounds__(PLAN_THREADS) void units_kernel(const PlanArgs pa) {
  __shared__ UnitsShared sh;
  plan_units<PLAN_THREADS>(pa, pa.plan.seq, sh);
}

hipError_t launch_units(const PlanArgs& pa, hipStream_t s) {
  hipLaunchKernelGGL(units_kernel, 1, PLAN_THREADS, 0, s, pa);
  return hipGetLastError();
}

hipError_t launch_ksteps(const AttnArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(ksteps_kernel, grid, WG_THREADS, 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_rowinfo_t(const AttnArgs& a, int dtype, bool cap, int grid,
                                   hipStream_t s) {
  if (dtype == DT_BF16) {
    if (cap) hipLaunchKernelGGL((rowinfo_kernel<BF16, D, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((rowinfo_kernel<BF16, D, false>), grid, WG_THREADS, 0, s, a);
  } else {
    if (cap) hipLaunchKernelGGL((rowinfo_kernel<F16, D, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((rowinfo_kernel<F16, D, false>), grid, WG_THREADS, 0, s, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void ticket_kernel(int* ticket) {
  if (threadIdx.x == 0) *ticket = 0;
}

hipError_t launch_ticket_reset(int* ticket, hipStream_t s) {
  hipLaunchKernelGGL(ticket_kernel, 1, 64, 0, s, ticket);
  return hipGetLastError();
}

hipError_t launch_rowinfo(const AttnArgs& a, int dtype, int d, bool cap, hipStream_t s) {
  const int64_t n = a.total_q * a.hq * 8;
  if (n <= 0) return hipSuccess;
  const int grid = (int)((n + WG_THREADS - 1) / WG_THREADS);
  switch (d) {
    case 64: return launch_rowinfo_t<64>(a, dtype, cap, grid, s);
    case 128: return launch_rowinfo_t<128>(a, dtype, cap, grid, s);
    default: return launch_rowinfo_t<160>(a, dtype, cap, grid, s);
  }
}

}  // namespace rga
