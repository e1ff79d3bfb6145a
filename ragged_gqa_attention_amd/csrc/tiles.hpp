// Global -> LDS staging of key tiles for the row-tile kernels (forward, dQ).
//
// A key tile holds KEY_STEP consecutive keys of one sequence.  Keys at or past
// the sequence end are written as zeros: the padding of the packed views is
// arbitrary (NaN in the tests), and 0 * NaN would poison the MFMA sums even
// where the softmax weight is exactly zero.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace rga {

constexpr int WG_THREADS = 256;
// Row-major key tile [KEY_STEP][LDK]: +8 halves keeps the 16-byte reads of 32
// consecutive rows on distinct LDS banks.
constexpr int LDK = HEAD_DIM + 8;
// Transposed key tile [HEAD_DIM][LDT]: +4 halves (34 dwords per row) keeps the
// 8-byte reads of 16 consecutive feature rows on distinct banks.
constexpr int LDT = KEY_STEP + 4;

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Row-major copy of keys [kbase, kbase + KEY_STEP) of a sequence starting at
// token k0 with Lk keys.  Consecutive threads take consecutive 16-byte chunks
// of a row, so each wave reads whole rows.
__device__ __forceinline__ void stage_keys_rowmajor(uint16_t* __restrict__ dst,
                                                    const uint16_t* __restrict__ src,
                                                    int64_t ts, int k0, int Lk, int kbase) {
  for (int t = threadIdx.x; t < KEY_STEP * CHUNKS; t += WG_THREADS) {
    const int key = t / CHUNKS;
    const int c = t - key * CHUNKS;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (kbase + key < Lk) val = load16(src + (int64_t)(k0 + kbase + key) * ts + c * 8);
    *reinterpret_cast<u32x4*>(dst + key * LDK + c * 8) = val;
  }
}

// Transposed copy dst[d][key] (stride LDT), optionally also the row-major copy
// into rm (stride LDK).  A task is a pair of keys times one 16-byte chunk, so
// each LDS write of the transposed tile is a full 32-bit word.
template <bool ALSO_ROWMAJOR>
__device__ __forceinline__ void stage_keys_transposed(uint16_t* __restrict__ dst,
                                                      uint16_t* __restrict__ rm,
                                                      const uint16_t* __restrict__ src,
                                                      int64_t ts, int k0, int Lk, int kbase) {
  constexpr int PAIRS = KEY_STEP / 2;
  for (int t = threadIdx.x; t < PAIRS * CHUNKS; t += WG_THREADS) {
    const int kp = t % PAIRS;
    const int c = t / PAIRS;
    const int key = 2 * kp;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (kbase + key < Lk) a = load16(src + (int64_t)(k0 + kbase + key) * ts + c * 8);
    if (kbase + key + 1 < Lk) b = load16(src + (int64_t)(k0 + kbase + key + 1) * ts + c * 8);
    uint16_t* col = dst + (c * 8) * LDT + key;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint32_t*>(col + (2 * e) * LDT) = interleave_lo(a[e], b[e]);
      *reinterpret_cast<uint32_t*>(col + (2 * e + 1) * LDT) = interleave_hi(a[e], b[e]);
    }
    if (ALSO_ROWMAJOR) {
      *reinterpret_cast<u32x4*>(rm + key * LDK + c * 8) = a;
      *reinterpret_cast<u32x4*>(rm + (key + 1) * LDK + c * 8) = b;
    }
  }
}

// A operand of a 32x32x16 product whose k index runs over keys of a transposed
// tile: lane (row l32 of the block, group g) takes keys {16s + 4g + 0..3,
// 16s + 8 + 4g + 0..3} of k-step s, matching the k order of an accumulator
// reused as B operand.
__device__ __forceinline__ u32x4 read_perm_a(const uint16_t* rowp) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(rowp + 8);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Logit x (base-2 units) from a raw dot product; also returns r = 1/(1+e^{2y})
// needed by the soft-cap derivative 1 - tanh^2 = 4 r (1 - r).
template <bool CAP>
__device__ __forceinline__ float logit2(float dot, float slope2, float dist, const LogitConsts& lc,
                                        float& r) {
  float t2;
  if (CAP) {
    r = fast_rcp(1.0f + fast_exp2(dot * lc.k_exp));
    t2 = __builtin_fmaf(lc.t_mul, r, lc.t_add);
  } else {
    r = 0.5f;
    t2 = dot * lc.s_lin;
  }
  return __builtin_fmaf(-slope2, __builtin_fabsf(dist), t2);
}

}  // namespace rga
