// Device planner, fixed-order K/V partial reduction, and the backward's row
// records for the standalone backward entry.
//
// The planner reads cu_q / cu_k on the device (no host synchronisation) and
// builds two work lists for the packed ragged batch (page "Noncausal Global
// Extreme-GQA Ragged Attention Full VJP", section "What You Have": 18-52
// sequences whose Q/K length ratio runs both ways):
//   * row tiles (forward, dQ): ceil(Lq * Hq / 128) per sequence, cost ~ Lk;
//   * key units (dK/dV): ceil(Lk / 128) key tiles per sequence, each split into
//     row chunks so that the whole batch yields about `target_units` units.
// Sequences are ranked by cost, largest first, so the longest work starts
// first.  A workgroup finds its item by binary search over the rank prefix.
#include "kernels.hpp"
#include "tiles.hpp"

namespace rga {

constexpr int PLAN_THREADS = 256;
constexpr int WG_THREADS = 256;          // reduce and row-record kernels
constexpr int PLAN_SORT_LIMIT = 8192;   // larger batches keep their natural order

__device__ __forceinline__ long long block_sum(long long v, long long* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = PLAN_THREADS / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const long long r = red[0];
  __syncthreads();
  return r;
}

// put(r, sum_{r' < r} count(r')) for r = 0..B.
template <class F, class G>
__device__ __forceinline__ void block_exclusive_scan(int B, F count, G put, int* part) {
  const int tid = threadIdx.x;
  const int seg = (B + PLAN_THREADS - 1) / PLAN_THREADS;
  const int lo = min(B, tid * seg), hi = min(B, lo + seg);
  int local = 0;
  for (int r = lo; r < hi; ++r) local += count(r);
  part[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < PLAN_THREADS; ++i) {
      const int c = part[i];
      part[i] = run;
      run += c;
    }
    put(B, run);
  }
  __syncthreads();
  int run = part[tid];
  for (int r = lo; r < hi; ++r) {
    put(r, run);
    run += count(r);
  }
  __syncthreads();
}

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const PlanArgs a) {
  __shared__ int bad;
  __shared__ long long red[PLAN_THREADS];
  __shared__ int part[PLAN_THREADS];
  const int tid = threadIdx.x;
  const int B = a.batch;
  int* seq = a.plan.seq;

  if (tid == 0) bad = 0;
  if (tid < 32) reinterpret_cast<u32x4*>(a.zero)[tid] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  for (int b = tid; b <= B; b += PLAN_THREADS) {
    const int cq = a.cu_q[b], ck = a.cu_k[b];
    bool fail = cq < 0 || (int64_t)cq > a.total_q || ck < 0 || (int64_t)ck > a.total_k;
    if (b == 0) fail |= (cq != 0) || (ck != 0);
    if (b == B) fail |= ((int64_t)cq != a.total_q) || ((int64_t)ck != a.total_k);
    if (b < B) fail |= (a.cu_q[b + 1] < cq) || (a.cu_k[b + 1] < ck);
    if (fail) bad = 1;   // benign race: every writer stores 1
  }
  __syncthreads();
  const bool ok = bad == 0;
  if (tid == 0) a.plan.flag[0] = ok ? 0 : 1;

  // Per-sequence extents; an invalid batch plans every sequence as empty.
  long long cost = 0;
  for (int b = tid; b < B; b += PLAN_THREADS) {
    const int q0 = ok ? a.cu_q[b] : 0, lq = ok ? a.cu_q[b + 1] - q0 : 0;
    const int k0 = ok ? a.cu_k[b] : 0, lk = ok ? a.cu_k[b + 1] - k0 : 0;
    const int rows = lq * a.hq;
    const int kt = (lk + KEY_TILE - 1) / KEY_TILE;
    int* s = seq + b * SEQ_FIELDS;
    s[SQ_Q0] = q0; s[SQ_LQ] = lq; s[SQ_K0] = k0; s[SQ_LK] = lk;
    s[SQ_ROWS] = rows; s[SQ_KTILES] = kt;
    cost += (long long)kt * rows;
  }
  const long long total_cost = block_sum(cost, red);
  long long target = (total_cost + a.target_units - 1) / a.target_units;
  if (target < a.min_chunk) target = a.min_chunk;
  target = (target + KV_ROW_STEP - 1) / KV_ROW_STEP * KV_ROW_STEP;
  for (int b = tid; b < B; b += PLAN_THREADS) {
    int* s = seq + b * SEQ_FIELDS;
    const long long rows = s[SQ_ROWS];
    int nchunk = 0, chunk = 0;
    if (rows > 0 && s[SQ_KTILES] > 0) {
      const long long n0 = (rows + target - 1) / target;
      long long len = (rows + n0 - 1) / n0;
      len = (len + KV_ROW_STEP - 1) / KV_ROW_STEP * KV_ROW_STEP;
      chunk = (int)len;
      nchunk = (int)((rows + len - 1) / len);
    }
    s[SQ_NCHUNK] = nchunk;
    s[SQ_CHUNK] = chunk;
  }
  __syncthreads();

  // Ranks: row tiles by Lk descending, key units by chunk length descending.
  for (int b = tid; b < B; b += PLAN_THREADS) {
    int rf = b, rk = b;
    if (B <= PLAN_SORT_LIMIT) {
      const int fb = seq[b * SEQ_FIELDS + SQ_LK], kb = seq[b * SEQ_FIELDS + SQ_CHUNK];
      rf = 0;
      rk = 0;
      for (int o = 0; o < B; ++o) {
        const int fo = seq[o * SEQ_FIELDS + SQ_LK], ko = seq[o * SEQ_FIELDS + SQ_CHUNK];
        rf += (fo > fb) || (fo == fb && o < b);
        rk += (ko > kb) || (ko == kb && o < b);
      }
    }
    a.plan.fwd_seq[rf] = b;
    a.plan.kv_seq[rk] = b;
    a.plan.kv_rank[b] = rk;
  }
  __syncthreads();

  const int hq = a.hq;
  block_exclusive_scan(B, [&](int r) {
    const int b = a.plan.fwd_seq[r];
    return (seq[b * SEQ_FIELDS + SQ_LQ] * hq + ROW_TILE - 1) / ROW_TILE;
  }, [&](int r, int v) { a.plan.fwd_off[r] = v; }, part);
  block_exclusive_scan(B, [&](int r) {
    const int b = a.plan.kv_seq[r];
    return seq[b * SEQ_FIELDS + SQ_KTILES] * seq[b * SEQ_FIELDS + SQ_NCHUNK];
  }, [&](int r, int v) { a.plan.kv_off[r] = v; }, part);
  // transposed 64-key tiles, in sequence order
  block_exclusive_scan(B, [&](int b) {
    return (seq[b * SEQ_FIELDS + SQ_LK] + TILE_ROWS - 1) / TILE_ROWS;
  }, [&](int b, int v) { if (b < B) seq[b * SEQ_FIELDS + SQ_TTOFF] = v; }, part);
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, 1, PLAN_THREADS, 0, s, a);
  return hipGetLastError();
}

// Transposed key tiles (see tt_key_pos): workgroup i writes tile i of K and of
// V, i.e. keys [64 j, 64 j + 64) of the sequence whose tiles start at or
// before i (j = i - first tile); keys past Lk become zeros.
__global__ __launch_bounds__(WG_THREADS) void transpose_keys_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t rows[TILE_ROWS][HEAD_DIM + 8];
  const int tile = blockIdx.x;
  const int* seq = a.plan.seq;
  if (a.batch <= 0) return;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq[mid * SEQ_FIELDS + SQ_TTOFF] <= tile) lo = mid; else hi = mid - 1;
  }
  const int* sb = seq + lo * SEQ_FIELDS;
  const int j = tile - sb[SQ_TTOFF];
  const int Lk = sb[SQ_LK];
  if (j < 0 || j * TILE_ROWS >= Lk) return;
  const int kbase = sb[SQ_K0] + j * TILE_ROWS;
  const int nkeys = min(TILE_ROWS, Lk - j * TILE_ROWS);
  const int tid = threadIdx.x;
  for (int t = 0; t < 2; ++t) {
    uint16_t* dst = t ? a.vt : a.kt;
    if (!dst) continue;    // uniform
    const uint16_t* src = t ? a.v : a.k;
    const int64_t ts = t ? a.v_ts : a.k_ts;
    for (int i = tid; i < TILE_ROWS * CHUNKS; i += WG_THREADS) {
      const int key = i / CHUNKS, c = i - key * CHUNKS;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < nkeys) x = load16(src + (int64_t)(kbase + key) * ts + c * 8);
      *reinterpret_cast<u32x4*>(&rows[key][c * 8]) = x;
    }
    __syncthreads();
    dst += (int64_t)tile * TILE_ELEMS;
    for (int o = tid; o < HEAD_DIM * (TILE_ROWS / 8); o += WG_THREADS) {
      const int d = o / (TILE_ROWS / 8), c = o - d * (TILE_ROWS / 8);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo16 = rows[tt_key_pos(8 * c + 2 * e)][d];
        const uint32_t hi16 = rows[tt_key_pos(8 * c + 2 * e + 1)][d];
        w[e] = lo16 | (hi16 << 16);
      }
      *reinterpret_cast<u32x4*>(dst + d * TILE_ROWS + c * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
  }
}

hipError_t launch_transpose_keys(const AttnArgs& a, int tiles, hipStream_t s) {
  if (tiles <= 0 || (!a.kt && !a.vt)) return hipSuccess;
  hipLaunchKernelGGL(transpose_keys_kernel, tiles, WG_THREADS, 0, s, a);
  return hipGetLastError();
}

// dK / dV of every key: sequences whose rows were split sum their FP32
// partials in chunk order; sequences without query rows get exact zeros;
// unsplit sequences were written by the dK/dV kernel and are skipped.
template <class T>
__global__ __launch_bounds__(WG_THREADS) void kv_reduce_kernel(const AttnArgs a) {
  constexpr int QUADS = HEAD_DIM / 4;
  const int64_t idx = (int64_t)blockIdx.x * WG_THREADS + threadIdx.x;
  if (idx >= a.total_k * QUADS) return;
  const int t = (int)(idx / QUADS);
  const int c4 = (int)(idx - (int64_t)t * QUADS);
  const int* seq = a.plan.seq;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq[mid * SEQ_FIELDS + SQ_K0] <= t) lo = mid; else hi = mid - 1;
  }
  const int* s = seq + lo * SEQ_FIELDS;
  const int lt = t - s[SQ_K0];
  const int nchunk = s[SQ_NCHUNK];
  f32x4 sk = {0.0f, 0.0f, 0.0f, 0.0f}, sv = {0.0f, 0.0f, 0.0f, 0.0f};
  if (lt < s[SQ_LK] && nchunk > 0) {
    if (nchunk == 1) return;
    const int kt = lt / KEY_TILE, kin = lt - kt * KEY_TILE;
    const int64_t base = (int64_t)a.plan.kv_off[a.plan.kv_rank[lo]] + (int64_t)kt * nchunk;
    for (int c = 0; c < nchunk; ++c) {
      const int64_t off = ((base + c) * KEY_TILE + kin) * HEAD_DIM + c4 * 4;
      sk += *reinterpret_cast<const f32x4*>(a.part_dk + off);
      sv += *reinterpret_cast<const f32x4*>(a.part_dv + off);
    }
  }
  *reinterpret_cast<u32x2*>(a.dk + (int64_t)t * a.dk_ts + c4 * 4) =
      u32x2{pack2<T>(sk[0], sk[1]), pack2<T>(sk[2], sk[3])};
  *reinterpret_cast<u32x2*>(a.dv + (int64_t)t * a.dv_ts + c4 * 4) =
      u32x2{pack2<T>(sv[0], sv[1]), pack2<T>(sv[2], sv[3])};
}

hipError_t launch_kv_reduce(const AttnArgs& a, int dtype, hipStream_t s) {
  const int64_t n = a.total_k * (HEAD_DIM / 4);
  if (n <= 0) return hipSuccess;
  const int grid = (int)((n + WG_THREADS - 1) / WG_THREADS);
  if (dtype == DT_BF16) hipLaunchKernelGGL(kv_reduce_kernel<BF16>, grid, WG_THREADS, 0, s, a);
  else hipLaunchKernelGGL(kv_reduce_kernel<F16>, grid, WG_THREADS, 0, s, a);
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
  const float slope2 = a.slopes[(int64_t)lo * a.slopes_stride + h] * LOG2E;
  const float moff = (CAP ? a.lc.t_add : 0.0f) - slope2 * (float)max(0, Lq - Lk - i);
  const float L = a.lse[r];
  const float negres = Lk > 0 ? moff - L * LOG2E : 0.0f;
  *reinterpret_cast<f32x4*>(a.rowinfo + r * 4) =
      f32x4{slope2, (float)max(i + Lk - Lq, 0), negres, acc};
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
