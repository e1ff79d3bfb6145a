// LDS tiles, operand reads and the logit pipeline shared by the gfx950 kernels.
//
// Every tile lives in LDS row-major (16-byte chunks of a 160-element row).  A
// product that contracts over the rows of a tile (P^T V, dS^T Q, P^T dO,
// dS K) reads its A operand with ds_read_b64_tr_b16, the CDNA4 transposing LDS
// read: inside each group of 16 lanes, lane i receives element i % 4 of the
// 8-byte words addressed by lanes 4e + i / 4 (e = 0..3).  So no transposed
// copy of any tile is ever written.
//
// Rows at or past a sequence's end are staged as zeros: the padding of the
// packed views is arbitrary (NaN in the tests) and 0 * NaN would poison MFMA
// sums even where the softmax weight is exactly zero.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace rga {

// Row stride of the LDS tiles read with 16-byte row reads (b128): 336 bytes puts
// the rows of each 8-lane phase on distinct 16-byte bank slots.
constexpr int LDK = HEAD_DIM + 8;
// Row stride of tiles read only through the transposing read: 352 bytes puts
// the four rows of each 16-lane group on distinct 32-byte bank slots.
constexpr int LDV = HEAD_DIM + 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// A operand of a 32x32x16 product that contracts over tile rows: lane
// (l32, g) receives X[r0 + 4g + 0..3][c0 + l32] and X[r0 + 8 + 4g + 0..3][c0 + l32],
// the k order of an accumulator (rows 8(r/4) + 4g + r%4) reused as B operand.
template <int LD>
__device__ __forceinline__ u32x4 read_tr_a(const uint16_t* X, int r0, int c0, int lane) {
  const int i = lane & 15;
  const int G = lane >> 4;
  const uint16_t* p = X + (r0 + 4 * (G >> 1) + (i >> 2)) * LD + c0 + 16 * (G & 1) + 4 * (i & 3);
  const u32x2 lo = read_tr(p);
  const u32x2 hi = read_tr(p + 8 * LD);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Row-major staging of up to two 160-wide sources into LDS through registers:
// load() issues the global reads for the next tile, store() writes them once
// the current tile's compute no longer needs the buffer.  Each thread owns
// PER_THREAD 16-byte chunks; rows [0, ROWS) come from source 0 and rows
// [ROWS, 2 ROWS) from source 1.
template <int THREADS, int ROWS>
struct PairStager {
  static constexpr int TASKS = 2 * ROWS * CHUNKS;
  static constexpr int PER_THREAD = TASKS / THREADS;
  static_assert(TASKS % THREADS == 0, "tile chunks must divide evenly over the threads");
  u32x4 reg[PER_THREAD];

  // rows of a key tile: row r of source s is token base + r, valid if r < valid
  __device__ __forceinline__ void load_keys(const uint16_t* s0, int64_t ts0, const uint16_t* s1,
                                            int64_t ts1, int64_t base, int valid) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * THREADS;
      const int which = t >= ROWS * CHUNKS;
      const int tt = t - which * ROWS * CHUNKS;
      const int r = tt / CHUNKS, c = tt - r * CHUNKS;
      const uint16_t* src = which ? s1 : s0;
      const int64_t ts = which ? ts1 : ts0;
      reg[u] = u32x4{0u, 0u, 0u, 0u};
      if (r < valid) reg[u] = load16(src + (base + r) * ts + c * 8);
    }
  }

  // rows of a folded (token, head) tile: folded row R = row0 + r, token R / hq,
  // head R % hq; valid if R < row_end
  __device__ __forceinline__ void load_rows(const uint16_t* s0, int64_t ts0, int64_t hs0,
                                            const uint16_t* s1, int64_t ts1, int64_t hs1,
                                            int q0, int hq, int row0, int row_end) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * THREADS;
      const int which = t >= ROWS * CHUNKS;
      const int tt = t - which * ROWS * CHUNKS;
      const int r = tt / CHUNKS, c = tt - r * CHUNKS;
      const int R = row0 + r;
      reg[u] = u32x4{0u, 0u, 0u, 0u};
      if (R < row_end) {
        const int tok = R / hq, h = R - tok * hq;
        reg[u] = which ? load16(s1 + (int64_t)(q0 + tok) * ts1 + (int64_t)h * hs1 + c * 8)
                       : load16(s0 + (int64_t)(q0 + tok) * ts0 + (int64_t)h * hs0 + c * 8);
      }
    }
  }

  template <int LD0, int LD1>
  __device__ __forceinline__ void store(uint16_t* d0, uint16_t* d1) const {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * THREADS;
      const int which = t >= ROWS * CHUNKS;
      const int tt = t - which * ROWS * CHUNKS;
      const int r = tt / CHUNKS, c = tt - r * CHUNKS;
      uint16_t* dst = which ? d1 + r * LD1 : d0 + r * LD0;
      *reinterpret_cast<u32x4*>(dst + c * 8) = reg[u];
    }
  }
};

// ---------------------------------------------------------------------------
// Swizzled row tiles filled by direct global->LDS loads.
//
// A tile of R rows x 160 16-bit features is stored without padding (320-byte
// rows, 20 chunks of 16 bytes) with the chunk index of row r XOR-ed with
// (r / 4) % 4.  LDS serves 16 lanes of a 16-byte read per pass from 16 chunk
// banks; rows r and r + 4k then start on different banks, so the 16 rows of a
// row read (one chunk each) and the 4 rows x 2 chunks of a transposing read
// both touch 16 distinct chunk banks.  The XOR only flips the two low bits of
// the chunk index, so a chunk never leaves its row.
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * HEAD_DIM + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// Logical (row, chunk) held by physical 16-byte slot `slot` of a swizzled tile.
__device__ __forceinline__ void swz_slot(int slot, int& row, int& chunk) {
  row = slot / CHUNKS;
  chunk = (slot - row * CHUNKS) ^ ((row >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// One wave-wide direct load: lane l copies the 16 bytes at `src` (its own
// address) to LDS at wave_dst + 16 l.  wave_dst must be the same for every lane.
__device__ __forceinline__ void load_lds16(const void* src, void* wave_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)const_cast<void*>(src), (lds_void_t*)wave_dst,
                                   16, 0, 0);
}

// Wait for this wave's outstanding global loads (direct LDS loads included).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// read_tr_a for a swizzled tile.
__device__ __forceinline__ u32x4 read_tr_swz(const uint16_t* X, int r0, int c0, int lane) {
  const int i = lane & 15;
  const int G = lane >> 4;
  const int row = r0 + 4 * (G >> 1) + (i >> 2);
  const int col = c0 + 16 * (G & 1) + 4 * (i & 3);
  const u32x2 lo = read_tr(X + swz_off(row, col >> 3) + (col & 7));
  const u32x2 hi = read_tr(X + swz_off(row + 8, col >> 3) + (col & 7));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Capped logit pieces from a raw dot product q.k (see LogitConsts):
//   r = 1 / (1 + e^{2 s / c}),   c tanh(s / c) log2(e) = t_add + t_mul * r,
// and 1 - tanh^2(s / c) = 4 r (1 - r).
__device__ __forceinline__ float cap_r(float dot, const LogitConsts& lc) {
  return fast_rcp(1.0f + fast_exp2(dot * lc.k_exp));
}

}  // namespace rga
