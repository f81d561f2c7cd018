// Row-major bf16 tiles in LDS, filled straight from global memory by
// global_load_lds_dwordx4 (no register staging), and the MFMA operand reads
// from them.
//
// A tile holds R token rows of D bf16 values (2D bytes, no padding). Row r is
// split into D/8 chunks of 16 bytes; logical chunk c of row r sits at physical
// chunk c ^ swz<D>(r). The permutation is chosen for the two read patterns
// the kernels use (ds_read_b128 serves 16 lanes per cycle and
// ds_read_b64_tr_b16 32 lanes, over 64 four-byte banks):
//   row reads  - lane (r, g) reads chunk c of row base + perm_row(r): the 16
//                lanes of a group touch rows {0..3, 16..19, 4..7, 20..23}
//                (+8), which swz spreads over distinct banks;
//   transposed - 32 lanes read 8 bytes each from 4 consecutive rows and four
//                consecutive chunks, which swz keeps on distinct banks.
#pragma once

#include "common.h"

namespace esm {

template <int D>
__device__ __forceinline__ int swz(int row) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b4 = (row >> 4) & 1;
  if (D == 16) return b4;
  if (D == 32) return b2 | (b4 << 1);
  if (D == 64) return b2 | (b4 << 1) | (b1 << 2);
  return b2 | (b4 << 1) | (b0 << 2) | (b1 << 3);  // D == 128
}

// Element offset of (row, first element of logical chunk c).
template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * D + 8 * (c ^ swz<D>(row));
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Waits until this wave's outstanding vector-memory operations (which include
// global_load_lds transfers into LDS) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Loads rows [0, R) of a tile whose row i is global row G + min(i, lim-1)*rs
// (rows past the valid range repeat the last valid one, lim >= 1) into the
// swizzled LDS tile T. The tile is written in 1 KB pieces, one
// global_load_lds_dwordx4 per wave and piece (lane l fills bytes 16l..16l+15
// of the piece); wave w of the 4 takes pieces w, w+4, ...
template <int D, int R>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ G, int rs, int lim,
                                          uint16_t* T, int w, int lane) {
  constexpr int NC = D / 8;
  constexpr int PIECES = R * NC / 64;
  static_assert(PIECES * 64 == R * NC, "tile must be a whole number of 1 KB pieces");
#pragma unroll
  for (int j = 0; j < (PIECES + 3) / 4; ++j) {
    const int i = w + 4 * j;
    if (PIECES % 4 == 0 || i < PIECES) {
      const int p = i * 64 + lane, row = p / NC, pc = p % NC;
      const int src_row = min(row, lim - 1);
      const uint16_t* src = G + src_row * rs + 8 * (pc ^ swz<D>(row));
      __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(T + i * 512), 16, 0, 0);
    }
  }
}

// Loads n <= 64 consecutive floats src[min(i, lim-1)], i < n, into LDS F[0..n)
// with one global_load_lds_dword by wave w_load (4 bytes per lane).
__device__ __forceinline__ void load_row_f32(const float* __restrict__ src, int n, int lim,
                                             float* F, int w, int w_load, int lane) {
  if (w == w_load && lane < n)
    __builtin_amdgcn_global_load_lds((gptr_t)(src + min(lane, lim - 1)), (lptr_t)F, 4, 0, 0);
}

// MFMA operand along d from a tile: lane (r, g) gets logical chunk c of row
// row (8 consecutive d values).
template <int D>
__device__ __forceinline__ u32x4 ld_row(const uint16_t* T, int row, int c) {
  return ld16(T + tile_off<D>(row, c));
}

// MFMA operand whose k index runs along the ROWS of the tile (the transposed
// tile): lane (r = l % 32, g = l / 32) receives T[k0 + 16g + e][col0 +
// perm_row(r)] for e = 0..7, through two ds_read_b64_tr_b16 (see ld_tr8 in
// common.h for the lane mapping of that instruction). k0 is a multiple of 8.
// ZERO_HI: lanes whose perm_row(r) >= ncols get zeros (tiles narrower than 32
// columns); their source addresses are clamped into the tile.
template <int D, bool ZERO_HI>
__device__ __forceinline__ u32x4 ld_tr_tile(const uint16_t* T, int k0, int col0, int ncols) {
  const int l = threadIdx.x & 63;
  const int s = l & 15, G = l >> 4, g = l >> 5;
  int col = perm_row(16 * (G & 1) + 4 * (s & 3));
  if (ZERO_HI && col >= ncols) col = 0;
  col += col0;
  const int row0 = k0 + 16 * g + (s >> 2), row1 = row0 + 4;
  const uint16_t* p0 = T + tile_off<D>(row0, col >> 3) + (col & 7);
  const uint16_t* p1 = T + tile_off<D>(row1, col >> 3) + (col & 7);
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
  const uint2 a = __builtin_bit_cast(uint2, v0), b = __builtin_bit_cast(uint2, v1);
  u32x4 out = {a.x, a.y, b.x, b.y};
  if (ZERO_HI && perm_row(l & 31) >= ncols) out = u32x4{0u, 0u, 0u, 0u};
  return out;
}

}  // namespace esm
