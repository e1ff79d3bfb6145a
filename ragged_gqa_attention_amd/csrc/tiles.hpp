// LDS tile layouts, direct global -> LDS copies, operand reads and the logit
// pipeline shared by the gfx950 kernels.
//
// Tiles are filled by direct loads (global_load_lds_dwordx4: one wave
// instruction copies 64 lanes x 16 bytes into 64 consecutive 16-byte LDS
// slots, so no staging registers are needed) and read without LDS bank
// conflicts.  LDS serves a 16-byte read 16 lanes at a time from 16 bank
// slots of 16 bytes (measured on gfx950: odd row strides in 16-byte units are
// conflict-free, a 320-byte stride is 4-way).
//
//  * Row tile: 64 rows (keys or folded query rows) x D features = D / 8 chunks
//    of 16 bytes per row (20 for D = 160), stored in blocks of 16 rows x 4
//    chunks (blk_off).
//    Read one chunk per lane ("row read", the A/B operand of a product that
//    contracts over features) or with the transposing read (the operand of a
//    product that contracts over rows).
//  * dS image (ds_off): a row tile with 64 keys as its rows and the 256
//    folded rows of a row tile as its columns, its key rows permuted inside
//    every 16-key group (tt_key_pos) in the order of the accumulator layout.
//
// Rows at or past a sequence's end are loaded from a zero block: the padding
// of the packed views is arbitrary (NaN in the tests) and 0 * NaN would poison
// MFMA sums even where the softmax weight is exactly zero.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace rga {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

constexpr int BLK_ELEMS = 64 * 8;                     // one 16-row x 4-chunk block

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ds_read_b64_tr_b16, the CDNA4 transposing LDS read: inside each group of 16
// lanes, lane i receives element i % 4 of the 8-byte words addressed by lanes
// 4e + i / 4 (e = 0..3).  Reading rows 4 (G/2) + i/4 and (+ 8) at features
// c0 + 16 (G%2) + 4 (i%4) (G = lane / 16) gives lane (l32, g) the A operand
// X^T[c0 + l32][r0 + 4g + 0..3, r0 + 8 + 4g + 0..3] of a 32x32x16 product that
// contracts over tile rows, in the k order of an accumulator reused as B.
__device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Element offset of chunk c of row r in a row tile: block (r / 16, c / 4)
// holds 64 consecutive slots, row-major inside, with the chunk's two low bits
// XOR-ed with (r / 4) % 4.  One wave load fills one block, reading 64
// contiguous bytes from each of 16 rows; a row read (16 lanes = 16
// consecutive rows of one chunk) and a transposing read (4 rows x 2 adjacent
// chunks) both touch 16 distinct bank slots.  A row spans Geo<D>::BLK_COLS
// blocks (D / 32).
template <int D>
__device__ __forceinline__ int blk_off(int r, int c) {
  constexpr int BC = Geo<D>::BLK_COLS;
  return (((r >> 4) * BC + (c >> 2)) * 64 + (r & 15) * 4 + ((c & 3) ^ ((r >> 2) & 3))) * 8;
}

// Key order of the accumulator layout reused as a B operand: the middle two
// quads of every 16-key group are swapped, so that lane half g of k-step s
// holds keys 16 s + {4g .. 4g + 3, 8 + 4g .. 8 + 4g + 3} (see common.hpp).
__device__ __forceinline__ int tt_key_pos(int k) {
  const int j = k & 15;
  const int q = j >> 2;
  return (k & ~15) | ((q == 1 ? 2 : q == 2 ? 1 : q) << 2) | (j & 3);
}

// Element offset of 16-byte chunk c (c = 0..31) of key k (0..63) in a dS
// image: the blocked row-tile layout of blk_off with 64 keys as its rows and
// ROW_TILE folded rows as its columns (eight block columns).  Chunk c holds
// rows 8c + {0..3, 8..11} or 8c - 4 + {0..3, 8..11}: inside every 16-row group
// the middle two quads are swapped (tt_key_pos), which is the row order of
// the dS accumulator registers.  A transposing read returns row
// 32 w + tt_key_pos(l32) to lane l32 of the wave that reads chunks 4w .. 4w + 3.
__device__ __forceinline__ int ds_off(int k, int c) {
  return (((k >> 4) * (ROW_TILE / 32) + (c >> 2)) * 64 + (k & 15) * 4 + ((c & 3) ^ ((k >> 2) & 3))) * 8;
}

// One wave-wide direct load: lane l copies the 16 bytes at `src` (its own
// address) to LDS at wave_dst + 16 l.  wave_dst must be the same for every lane.
__device__ __forceinline__ void load_lds16(const void* src, void* wave_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)const_cast<void*>(src), (lds_void_t*)wave_dst,
                                   16, 0, 0);
}

// The same copy, issued where the compiler does not see it.  The compiler
// orders every LDS read it cannot tell apart from a pending direct load after
// that load (and, as vector memory operations complete in issue order, after
// everything issued before it), which defeats a prefetch into one buffer of a
// ring while another is being read.  Callers of this form must themselves
// wait (wait_vm / wait_vm_le, then a barrier) before any wave reads the bytes.
__device__ __forceinline__ void load_lds16_unseen(const void* src, void* wave_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_void_t*)wave_dst);
  // M0 holds the LDS base of the copy; one wait state between the M0 write
  // and the copy that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "m0");
}

// Wait for this wave's outstanding global loads (direct LDS loads included).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order for this count).
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 16, "vmcnt field holds 0..15 in its low bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Copies the blocked row tile of rows [row0, row0 + 64) of a strided
// [tokens, D] view (rows past `nrows` read `zero`) with four waves: wave
// group w (0..3) copies rows 16 w .. 16 w + 15, lane l holding row
// 16 w + l / 4 for all D / 32 of its loads.  UNSEEN: issue them as
// load_lds16_unseen.
template <int D, bool UNSEEN = false>
__device__ __forceinline__ void load_row_tile(uint16_t* tile, const uint16_t* src, int64_t ts,
                                              int row0, int nrows, const uint16_t* zero,
                                              int w, int lane) {
  constexpr int BC = Geo<D>::BLK_COLS;
  const int r = 16 * w + (lane >> 2);
  const int c = (lane & 3) ^ ((lane >> 4) & 3);
  const bool ok = row0 + r < nrows;
  const uint16_t* p = (ok ? src + (int64_t)(row0 + r) * ts : zero) + c * 8;
#pragma unroll
  for (int b = 0; b < BC; ++b) {
    if (UNSEEN) load_lds16_unseen(p + b * 32, tile + (w * BC + b) * BLK_ELEMS);
    else load_lds16(p + b * 32, tile + (w * BC + b) * BLK_ELEMS);
  }
}

// Capped logit pieces from a raw dot product q.k (see LogitConsts):
//   r = 1 / (1 + e^{2 s / c}),   c tanh(s / c) log2(e) = t_add + t_mul * r,
// and 1 - tanh^2(s / c) = 4 r (1 - r).
__device__ __forceinline__ float cap_r(float dot, const LogitConsts& lc) {
  return fast_rcp(1.0f + fast_exp2(dot * lc.k_exp));
}

}  // namespace rga
