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
#include "kernels.hpp"
#include "planner.hpp"
#include "tiles.hpp"

namespace rga {

constexpr int PLAN_THREADS = 256;
constexpr int WG_THREADS = 256;          // row-record kernel

constexpr int PLAN_WAVES = PLAN_THREADS / 64;

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

__device__ __forceinline__ void plan_block(const PlanArgs& a) {
  __shared__ long long red[PLAN_WAVES];
  __shared__ int part[PLAN_WAVES];
  __shared__ int l_seq[PLAN_LDS_B * SEQ_FIELDS];
  __shared__ int l_hw[PLAN_LDS_HEADS];
  __shared__ int l_class[PLAN_COST_CLASSES + 1], l_foff_c[PLAN_COST_CLASSES];
  __shared__ int l_tseq[PLAN_LDS_TILES];
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int hq = a.hq;
  const bool in_lds = B <= PLAN_LDS_B;
  int* seq = in_lds ? l_seq : a.plan.seq;

  if (tid < 32) reinterpret_cast<u32x4*>(a.zero)[tid] = u32x4{0u, 0u, 0u, 0u};
  // the slopes, requested first (their loads overlap those of the checks
  // below); thread tid takes (sequence, head) pairs tid + 256 k
  constexpr int SPER = PLAN_LDS_HEADS / PLAN_THREADS;
  const bool hw_lds = (long long)B * hq <= PLAN_LDS_HEADS;
  const int sb0 = tid / hq, sh0 = tid - sb0 * hq;   // pair tid
  const int sdb = PLAN_THREADS / hq, sdh = PLAN_THREADS - sdb * hq;
  float sv[SPER];
  {
    int b = sb0, h = sh0;
#pragma unroll
    for (int k = 0; k < SPER; ++k) {
      sv[k] = hw_lds && b < B ? a.slopes[(int64_t)b * a.slopes_stride + h] : 0.0f;
      b += sdb;
      h += sdh;
      if (h >= hq) { h -= hq; ++b; }
    }
  }
  // checks of cu_q / cu_k and the per-sequence extents in one pass; an
  // invalid batch is then planned with every sequence empty
  auto extents = [&](int b, int q0, int lq, int k0, int lk) {
    int* s = seq + b * SEQ_FIELDS;
    s[SQ_Q0] = q0; s[SQ_LQ] = lq; s[SQ_K0] = k0; s[SQ_LK] = lk;
    s[SQ_ROWS] = lq * a.hq;
    s[SQ_KTILES] = (lk + KEY_TILE - 1) / KEY_TILE;
    // n / Lq = (umulhi(n, mul) + n) >> shift (see fast_div)
    uint32_t sh = 0;
    while (lq > 0 && (1u << sh) < (uint32_t)lq) ++sh;
    s[SQ_LQSHIFT] = (int)sh;
    s[SQ_LQMUL] = lq > 0 ? (int)(uint32_t)((((1ull << sh) - (uint64_t)lq) << 32) / (uint64_t)lq + 1) : 0;
  };
  bool bad = false;
  for (int b = tid; b <= B; b += PLAN_THREADS) {
    const int cq = a.cu_q[b], ck = a.cu_k[b];
    const int nq = b < B ? a.cu_q[b + 1] : cq, nk = b < B ? a.cu_k[b + 1] : ck;
    bool fail = cq < 0 || (int64_t)cq > a.total_q || ck < 0 || (int64_t)ck > a.total_k;
    if (b == 0) fail |= (cq != 0) || (ck != 0);
    if (b == B) fail |= ((int64_t)cq != a.total_q) || ((int64_t)ck != a.total_k);
    if (b < B) fail |= (nq < cq) || (nk < ck);
    bad |= fail;
    // (a failed check leaves this sequence empty, so no length is negative)
    if (b < B) {
      if (fail) extents(b, 0, 0, 0, 0);
      else extents(b, cq, nq - cq, ck, nk - ck);
    }
  }
  const bool ok = __syncthreads_or(bad) == 0;
  if (tid == 0) a.plan.flag[0] = ok ? 0 : 1;
  if (!ok) {
    for (int b = tid; b < B; b += PLAN_THREADS) extents(b, 0, 0, 0, 0);
    __syncthreads();
  }

  // 256-row tiles in batch order (their key-step ranges are kept in this
  // order); tile -> sequence in LDS when the tiles fit
  block_exclusive_scan<PLAN_THREADS>(B, [&](int b) {
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
    for (int i0 = 0; i0 < B * hq; i0 += PLAN_THREADS * PER) {
      float v[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = i0 + k * PLAN_THREADS + tid;
        const int b = i / hq;
        v[k] = i < B * hq ? a.slopes[(int64_t)b * a.slopes_stride + (i - b * hq)] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = i0 + k * PLAN_THREADS + tid;
        if (i < B * hq)
          hw[i] = key_half_width(v[k] * LOG2E, seq[(i / hq) * SEQ_FIELDS + SQ_LK], a.skip_log2);
      }
    }
  }
  for (int i = tid; i <= PLAN_COST_CLASSES; i += PLAN_THREADS) l_class[i] = 0;
  __threadfence_block();
  __syncthreads();
  auto seq_of_tile = [&](int g) {
    if (g < PLAN_LDS_TILES) return l_tseq[g];
    return last_at_most(B, g, [&](int x) { return seq[x * SEQ_FIELDS + SQ_RTOFF]; });
  };
  for (int g = tid; g < nrt; g += PLAN_THREADS) {
    const int b = seq_of_tile(g);
    const int* s = seq + b * SEQ_FIELDS;
    int lo, hi;
    tile_key_steps(s, g - s[SQ_RTOFF], hw + b * hq, lo, hi);
    a.ksteps[2 * g] = lo;
    a.ksteps[2 * g + 1] = hi;
    // class 0 holds the longest tiles
    atomicAdd(&l_class[PLAN_COST_CLASSES - 1 - min(hi - lo, PLAN_COST_CLASSES - 1)], 1);
  }
  __syncthreads();
  // workgroup -> row tile, longest first; entries past the last tile get
  // sequence -1
  block_exclusive_scan<PLAN_THREADS>(PLAN_COST_CLASSES, [&](int c) { return l_class[c]; },
                                     [&](int c, int v) { if (c < PLAN_COST_CLASSES) l_foff_c[c] = v; },
                                     part);
  for (int g = tid; g < nrt; g += PLAN_THREADS) {
    const int lo = a.ksteps[2 * g], hi = a.ksteps[2 * g + 1];
    const int pos = atomicAdd(&l_foff_c[PLAN_COST_CLASSES - 1 - min(hi - lo, PLAN_COST_CLASSES - 1)], 1);
    const int b = seq_of_tile(g);
    a.plan.fwd_map[2 * pos] = b;
    a.plan.fwd_map[2 * pos + 1] = g - seq[b * SEQ_FIELDS + SQ_RTOFF];
  }
  for (int i = nrt + tid; i < a.fwd_slots; i += PLAN_THREADS) {
    a.plan.fwd_map[2 * i] = -1;
    a.plan.fwd_map[2 * i + 1] = 0;
  }
  if (tid == 0) a.plan.kv_head[2] = nrt;
  // transposed 64-key tiles, in sequence order
  block_exclusive_scan<PLAN_THREADS>(B, [&](int b) {
    return (seq[b * SEQ_FIELDS + SQ_LK] + TILE_ROWS - 1) / TILE_ROWS;
  }, [&](int b, int v) { if (b < B) seq[b * SEQ_FIELDS + SQ_TTOFF] = v; }, part);
  // 128-key tiles in batch order (dK / dV units and partial sums walk them)
  block_exclusive_scan<PLAN_THREADS>(B, [&](int b) { return seq[b * SEQ_FIELDS + SQ_KTILES]; },
                       [&](int b, int v) { if (b < B) seq[b * SEQ_FIELDS + SQ_KTOFF] = v; }, part);
  // stored dS images, in sequence order, while they fit the workspace (a
  // sequence that does not fit recomputes dS in the dQ kernel)
  auto images = [&](int b) -> long long {
    const int* sb = seq + b * SEQ_FIELDS;
    if (sb[SQ_ROWS] == 0 || sb[SQ_LK] == 0) return 0;
    return (long long)((sb[SQ_ROWS] + ROW_TILE - 1) / ROW_TILE) *
           ((sb[SQ_LK] + TILE_ROWS - 1) / TILE_ROWS);
  };
  block_exclusive_scan<PLAN_THREADS>(B, images, [&](int b, long long off) {
    if (b < B) {
      const long long n = images(b);
      seq[b * SEQ_FIELDS + SQ_DSOFF] = (n > 0 && off + n <= a.ds_images) ? (int)off : -1;
    }
  }, red);

  if (in_lds) {   // the kernels read the plan from global memory
    for (int i = tid; i < B * SEQ_FIELDS; i += PLAN_THREADS) a.plan.seq[i] = l_seq[i];
  }
}

// Transposed key tile `tile` of K (see tt_key_pos; read by the dQ kernel):
// keys [64 j, 64 j + 64) of the sequence whose tiles start at or
// before `tile` (j = tile - first tile, tiles counted as in the planner's
// SQ_TTOFF); keys past Lk become zeros.  The sequence is found from cu_k
// directly, so this runs alongside the planner: wave 0 checks cu_k and scans
// the per-sequence tile counts with lane shuffles (lane l owns a contiguous
// run of sequences).  An invalid cu_k (which the planner flags, and which
// then plans no work) transposes nothing.
__device__ __forceinline__ void transpose_tiles(const PlanArgs& pa, const AttnArgs& a, int tile) {
  __shared__ __attribute__((aligned(16))) uint16_t rows[TILE_ROWS][HEAD_DIM + 8];
  __shared__ int s_b, s_j;
  const int B = pa.batch;
  if (!a.kt || B <= 0) return;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const int seg = (B + 63) / 64;
    const int lo = min(B, lane * seg), hi = min(B, lo + seg);
    bool fail = false;
    int count = 0;
    int prev = lo <= B ? pa.cu_k[lo] : 0;
    if (lo == 0) fail |= prev != 0;
    fail |= prev < 0 || (int64_t)prev > pa.total_k;
    for (int b = lo; b < hi; ++b) {
      const int nx = pa.cu_k[b + 1];
      fail |= nx < prev || (int64_t)nx > pa.total_k;
      count += (nx - prev + TILE_ROWS - 1) / TILE_ROWS;
      prev = nx;
    }
    if (hi == B && lo < hi) fail |= (int64_t)prev != pa.total_k;
    if (B <= lane * seg && lane * seg < B + seg) fail |= (int64_t)pa.cu_k[B] != pa.total_k;
    const bool any_fail = __any(fail);
    int x = count;   // inclusive scan over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    int run = x - count;   // tiles before this lane's first sequence
    int fb = -1, fj = 0;
    if (!any_fail && run <= tile && tile < x) {
      for (int b = lo; b < hi; ++b) {
        const int n = (pa.cu_k[b + 1] - pa.cu_k[b] + TILE_ROWS - 1) / TILE_ROWS;
        if (tile < run + n) { fb = b; fj = tile - run; break; }
        run += n;
      }
    }
    const unsigned long long who = __ballot(fb >= 0);
    if (lane == 0) { s_b = -1; s_j = 0; }
    if (who != 0 && lane == __ffsll((long long)who) - 1) { s_b = fb; s_j = fj; }
  }
  __syncthreads();
  const int b = s_b, j = s_j;
  if (b < 0) return;
  const int k0 = pa.cu_k[b];
  const int Lk = pa.cu_k[b + 1] - k0;
  const int kbase = k0 + j * TILE_ROWS;
  const int nkeys = min(TILE_ROWS, Lk - j * TILE_ROWS);
  {
    for (int i = tid; i < TILE_ROWS * CHUNKS; i += PLAN_THREADS) {
      const int key = i / CHUNKS, c = i - key * CHUNKS;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < nkeys) x = load16(a.k + (int64_t)(kbase + key) * a.k_ts + c * 8);
      *reinterpret_cast<u32x4*>(&rows[key][c * 8]) = x;
    }
    __syncthreads();
    uint16_t* dst = a.kt + (int64_t)tile * TILE_ELEMS;
    // task: feature pair (2 dp, 2 dp + 1) x chunk c of 8 keys
    for (int o = tid; o < (HEAD_DIM / 2) * (TILE_ROWS / 8); o += PLAN_THREADS) {
      const int dp = o / (TILE_ROWS / 8), c = o - dp * (TILE_ROWS / 8);
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x0 = *reinterpret_cast<const uint32_t*>(&rows[tt_key_pos(8 * c + 2 * e)][2 * dp]);
        const uint32_t x1 =
            *reinterpret_cast<const uint32_t*>(&rows[tt_key_pos(8 * c + 2 * e + 1)][2 * dp]);
        w0[e] = interleave_lo(x0, x1);
        w1[e] = interleave_hi(x0, x1);
      }
      *reinterpret_cast<u32x4*>(dst + (2 * dp) * TILE_ROWS + c * 8) = u32x4{w0[0], w0[1], w0[2], w0[3]};
      *reinterpret_cast<u32x4*>(dst + (2 * dp + 1) * TILE_ROWS + c * 8) =
          u32x4{w1[0], w1[1], w1[2], w1[3]};
    }
    __syncthreads();
  }
}

// Workgroup 0 plans; workgroup 1 + i transposes key tile i of K and V.
__global__ __launch_bounds__(PLAN_THREADS) void prep_kernel(const PlanArgs pa, const AttnArgs a) {
  if (blockIdx.x == 0) plan_block(pa);
  else transpose_tiles(pa, a, blockIdx.x - 1);
}

hipError_t launch_prep(const PlanArgs& pa, const AttnArgs& a, int key_tiles, hipStream_t s) {
  const int transposers = a.kt ? key_tiles : 0;
  hipLaunchKernelGGL(prep_kernel, 1 + transposers, PLAN_THREADS, 0, s, pa, a);
  return hipGetLastError();
}

// Row records for the backward entry that starts from a saved forward:
// Delta = sum_d dout[row, d] * out[row, d] over the stored 16-bit output, the
// slope in base-2 units, the clamped ALiBi centre and the base-2 residual of
// the stored natural-log L relative to the row offset the forward used (see
// fwd.hip).  Eight lanes share a row; each reads 16-byte chunks.
template <class T, bool CAP>
__global__ __launch_bounds__(WG_THREADS) void rowinfo_kernel(const AttnArgs a) {
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
  // sequence of token t: the last b with q0(b) <= t (never an empty one)
  const int* seq = a.plan.seq;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq[mid * SEQ_FIELDS + SQ_Q0] <= t) lo = mid; else hi = mid - 1;
  }
  const int* s = seq + lo * SEQ_FIELDS;
  const int i = (int)(t - s[SQ_Q0]);
  const int Lq = s[SQ_LQ], Lk = s[SQ_LK];
  const int64_t fr = (int64_t)s[SQ_Q0] * a.hq + (int64_t)h * Lq + i;   // folded row record
  const float slope2 = a.slopes[(int64_t)lo * a.slopes_stride + h] * LOG2E;
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)max(0, Lq - Lk - i);
  const float L = a.lse[r];
  const float negres = Lk > 0 ? moff - L * LOG2E : 0.0f;
  *reinterpret_cast<f32x4*>(a.rowinfo + fr * 4) =
      f32x4{slope2, (float)max(i + Lk - Lq, 0), negres, acc};
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
    const f32x4 info =
        *reinterpret_cast<const f32x4*>(a.rowinfo + ((int64_t)sq[SQ_Q0] * a.hq + R) * 4);
    slope2 = info[0];
    centre = (int)info[1];
    const float radd = info[2];   // added to every exponent of the row
    if (a.skip_log2 > 0.0f && __builtin_isfinite(radd))
      thr = SKIP_UNDERFLOW + __builtin_fmaxf(radd, 0.0f);
  }
  int lo, hi;
  row_key_steps(ok, slope2, centre, Lk, thr, lo, hi);
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

hipError_t launch_rowinfo(const AttnArgs& a, int dtype, bool cap, hipStream_t s) {
  const int64_t n = a.total_q * a.hq * 8;
  if (n <= 0) return hipSuccess;
  const int grid = (int)((n + WG_THREADS - 1) / WG_THREADS);
  if (dtype == DT_BF16) {
    if (cap) hipLaunchKernelGGL((rowinfo_kernel<BF16, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((rowinfo_kernel<BF16, false>), grid, WG_THREADS, 0, s, a);
  } else {
    if (cap) hipLaunchKernelGGL((rowinfo_kernel<F16, true>), grid, WG_THREADS, 0, s, a);
    else hipLaunchKernelGGL((rowinfo_kernel<F16, false>), grid, WG_THREADS, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace rga
