// Device-side building blocks shared by the gfx950 attention kernels.
//
// Tile geometry.  Every kernel works with wave64 and the CDNA4 instruction
// v_mfma_f32_32x32x16_{f16,bf16}: D[32x32] += A[32x16] * B[16x32] with FP32
// accumulation.  Operand layout (per lane l, l32 = l % 32, g = l / 32):
//   A: lane holds A[l32][8g .. 8g+7]      (row l32, eight consecutive k)
//   B: lane holds B[8g .. 8g+7][l32]      (column l32, eight consecutive k)
//   D: lane holds D[8(r/4) + 4g + r%4][l32] in accumulator register r = 0..15
// A head dimension D of 64, 128 or 160 is D / 16 k-steps of 16 (ten for 160),
// so no padding of the feature axis is needed.
//
// When a result tile D is reused as a B operand of the next product (P or dS
// feeding PV / dQ / dK / dV), the sixteen k-values a lane owns are not the
// canonical 8g..8g+7 but {16s + 4g + 0..3, 16s + 8 + 4g + 0..3} for k-step
// s = 0, 1.  The matching A operand is read in the same order with the
// transposing LDS read (see read_tr), so the contraction is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rga {

// Feature-axis geometry of head dimension D (64, 128 or 160).
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128 || D == 160, "head dimension 64, 128 or 160");
  static constexpr int KSTEPS = D / 16;     // k-steps of the QK^T / dO V^T products
  static constexpr int DBLK = D / 32;       // 32-wide feature blocks of O, dQ, dK, dV
  static constexpr int CHUNKS = D / 8;      // 16-byte chunks per row
  static constexpr int BLK_COLS = CHUNKS / 4;   // 4-chunk blocks across a row (tiles.hpp)
};
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct F16 {};
struct BF16 {};

// Compile-time flag passed to generic lambdas (e.g. a masked and an unmasked
// instance of one loop body).
template <bool B> struct Flag { static constexpr bool value = B; };

template <class T> __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <> __device__ __forceinline__ f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values (round to nearest even), lo in bits 0..15.
template <class T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-bit value (low or high half of a word) -> float.
template <class T> __device__ __forceinline__ float lo_f(uint32_t w);
template <class T> __device__ __forceinline__ float hi_f(uint32_t w);
template <> __device__ __forceinline__ float lo_f<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <> __device__ __forceinline__ float hi_f<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}
template <> __device__ __forceinline__ float lo_f<BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
template <> __device__ __forceinline__ float hi_f<BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// acc + (lo + hi) of a packed pair of 16-bit values, as one v_dot2 with ones.
template <class T> __device__ __forceinline__ float add_pair(uint32_t w, float acc);
template <> __device__ __forceinline__ float add_pair<F16>(uint32_t w, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}
template <> __device__ __forceinline__ float add_pair<BF16>(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (l ^ 32): the other half of a 32x32 accumulator column pair.
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32, 64); }

// Word k of the pair-interleave of two packed 16-bit rows: (a.e, b.e) for
// element e = 2k + hi.
__device__ __forceinline__ uint32_t interleave_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t interleave_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Constants of the logit pipeline, in base-2 units so the softmax uses exp2:
//   x = log2(e) * (c * tanh(s / c) - slope * |i + Lk - Lq - j|)
// with s = sigma * <q, k> and tanh(y) = 1 - 2 / (1 + e^{2y}).
struct LogitConsts {
  float k_exp;    // e^{2 s / c} = exp2(k_exp * dot),   k_exp = 2 sigma log2(e) / c
  float t_mul;    // x_cap = t_mul * 1/(1 + e^{2y}) + t_add
  float t_add;    //   t_mul = -2 c log2(e),  t_add = c log2(e)
  float s_lin;    // uncapped: x = s_lin * dot,  s_lin = sigma log2(e)
  float sigma;    // scale_multiplier / sqrt(head_dim)
};

// Per-sequence facts written by the planner (int32 each, SEQ_FIELDS per
// sequence).  A "sequence" of the plan is one (packed sequence b, K/V head g)
// pair, v = b * hkv + g: the rows of the group = hq / hkv query heads that share
// K/V head g fold into its M dimension (row R = h * Lq + i, h local to the group).
enum SeqField {
  SQ_Q0 = 0, SQ_LQ, SQ_K0, SQ_LK, SQ_ROWS,
  SQ_KTILES,  // 128-key tiles of the sequence (dK/dV)
  SQ_DSOFF,   // first stored dS image of the sequence, -1 when its dS is not stored
  SQ_KTOFF,   // first 128-key tile of the sequence in batch order (prefix of SQ_KTILES)
  SQ_LQMUL,   // fast_div constants of Lq (folded rows are head-major, see unfold_row)
  SQ_LQSHIFT,
  SQ_RTOFF,   // first 256-row tile of the sequence in batch order (prefix of row tiles)
  SQ_HB,      // first query head of the sequence's head group (g * group)
  SQ_G,       // its K/V head g
  SEQ_FIELDS
};

// Fields of a 128-key tile's record for the dK/dV work split (int32 each,
// KV_FIELDS per key tile, batch order): the key tile, its share of the
// flattened visit list, and copies of its sequence's record so a workgroup
// reads everything with one load.
enum KvField {
  KV_B = 0,    // sequence
  KV_KTILE,    // 128-key tile of the sequence
  KV_V,        // 64-row steps of the row tiles that visit the key tile
  KV_S,        // first of its items in the work list (see plan_units)
  KV_Q0, KV_K0, KV_LK, KV_ROWS, KV_RTOFF, KV_DSOFF, KV_LQ, KV_LQMUL, KV_LQSHIFT,
  KV_HB, KV_G,   // first query head of the group, K/V head
  KV_PAD0,
  KV_FIELDS
};

// Work lists built on the device; all arrays live in the caller's workspace.
struct Plan {
  int* seq;        // [B * SEQ_FIELDS]
  int* flag;       // [4]    [0] = 1 when cu_q / cu_k failed validation,
                   //        [2] the forward's tile ticket (AttnArgs::fwd_ticket)
  // Row-tile workgroup i -> (sequence, tile in sequence), longest tiles first,
  // (-1, 0) past the last tile; a workgroup finds its tile with one load.
  int* fwd_map;    // [fwd_slots * 2]
  // dK/dV work split (see plan_units): a record per 128-key tile (KvField),
  // each workgroup's first key tile (-1: empty share); kv_head holds W, the
  // number of key tiles, the number of row tiles and the segment items.
  int* ktab;       // [key tiles * KV_FIELDS]
  int* wg_first;   // [kv_wgs]
  int* kv_head;    // [4]
};

// n / d for 0 <= n < 2^31 with a host-computed multiplier (round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): shift = ceil(log2 d), mul = floor(2^32 (2^shift - d) / d) + 1.
__device__ __forceinline__ int fast_div(int n, uint32_t mul, uint32_t shift) {
  return (int)((__umulhi((uint32_t)n, mul) + (uint32_t)n) >> shift);
}

// fast_div constants of d >= 0 (d = 0 gives zeros; nothing divides by it):
// n / d = (umulhi(n, mul) + n) >> shift.
__device__ __forceinline__ void fast_div_consts(int d, uint32_t& mul, uint32_t& shift) {
  uint32_t sh = 0;
  while (d > 0 && (1u << sh) < (uint32_t)d) ++sh;
  shift = sh;
  mul = d > 0 ? (uint32_t)((((1ull << sh) - (uint64_t)d) << 32) / (uint64_t)d + 1) : 0u;
}

// Folded row R of a sequence -> (token i, head h).  The Lq x Hq rows are
// folded head-major, R = h * Lq + i: the rows of a tile share few heads, hence
// similar ALiBi slopes.  sq: the sequence's planner record.
__device__ __forceinline__ void unfold_row(int R, int lq, uint32_t mul, uint32_t shift, int& i,
                                           int& h) {
  h = fast_div(R, mul, shift);
  i = R - h * lq;
}
__device__ __forceinline__ void unfold_row(int R, const int* sq, int& i, int& h) {
  unfold_row(R, sq[SQ_LQ], (uint32_t)sq[SQ_LQMUL], (uint32_t)sq[SQ_LQSHIFT], i, h);
}

}  // namespace rga
