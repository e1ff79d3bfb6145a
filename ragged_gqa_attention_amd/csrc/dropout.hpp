// Counter-based dropout (page "python-20261012-ragged-flash-attention-
// gradient-recompute", section "Root causes addressed": a splitmix64 hash of
// (seed, b, h, row, col), so every pass rebuilds the same mask whatever its
// tiling; one rate or one per row).
//
// splitmix64 (Steele, Lea and Flood 2014) returns mix64(x + n gamma) as its
// n-th output from state x.  The (packed sequence b, query head h) stream has
// state K = output b * 2^16 + h + 1 of the generator started at the seed; the
// word of local row i and local key j is output i * 2^32 + j + 1 of that
// stream, mix64(A_i + gamma j) with A_i = K + gamma (i * 2^32 + 1).  Key j is
// kept iff the word's top 32 bits reach T = floor(p * 2^32), and a kept
// weight is scaled by 1 / (1 - p).
//
// Each row's A_i, T and scale form a 16-byte record (drop_row); the inner
// loops add gamma j (or gamma times a step's first key plus a per-register
// constant) and run the output function.
#pragma once

#include "kernels.hpp"

namespace rga {

constexpr uint64_t SM_GAMMA = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t sm_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Top 32 bits of the word at counter z (the final xor-shift only moves bits
// down, so they come from the product's high half alone).
__device__ __forceinline__ uint32_t sm_word_hi(uint64_t z) {
  return (uint32_t)(sm_mix64(z) >> 32);
}

// The dropout record of (packed sequence b, query head h, local row i): the
// counter base A_i, the threshold and the scale (float bits).
__device__ __forceinline__ u32x4 drop_row(const AttnArgs& a, int b, int h, int i, int64_t token) {
  const uint64_t n = ((uint64_t)(uint32_t)b << 16) + (uint64_t)(uint32_t)h + 1;
  const uint64_t K = sm_mix64(a.drop_seed + n * SM_GAMMA);
  const uint64_t A = K + SM_GAMMA * (((uint64_t)(uint32_t)i << 32) + 1);
  uint32_t thr = a.drop_thr;
  float scale = a.drop_scale;
  if (a.drop_rates) {
    // clamped to [0, 1 - 2^-24]; floor(p * 2^32) and 1 / (1 - p) are exact /
    // correctly rounded in double, as on the host
    const float p = __builtin_fminf(__builtin_fmaxf(a.drop_rates[token * a.hq + h], 0.0f),
                                    0.99999994f);
    thr = (uint32_t)__builtin_floor((double)p * 4294967296.0);
    scale = (float)(1.0 / (1.0 - (double)p));
  }
  return u32x4{(uint32_t)A, (uint32_t)(A >> 32), thr, __builtin_bit_cast(uint32_t, scale)};
}

__device__ __forceinline__ uint64_t drop_base(const u32x4& r) {
  return (uint64_t)r[0] | ((uint64_t)r[1] << 32);
}

// The record's scale.  The element goes through a scalar first: this
// compiler lowers __builtin_bit_cast of an ext_vector element (v[3]) to a
// cast of element 0.
__device__ __forceinline__ float drop_scale_of(const u32x4& r) {
  const uint32_t bits = r[3];
  return __builtin_bit_cast(float, bits);
}

// Whether key offset j (from the record's row) is kept.
__device__ __forceinline__ bool drop_keep(uint64_t base, uint32_t j, uint32_t thr) {
  return sm_word_hi(base + SM_GAMMA * (uint64_t)j) >= thr;
}

}  // namespace rga
