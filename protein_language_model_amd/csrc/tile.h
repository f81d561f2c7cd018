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

// Stores the two rotary halves of 8 pairs of tile row `row` (logical chunks c
// and c + D/16, c < D/16) with two ds_write_b128. On gfx950 one cycle of a
// 16-byte LDS write serves 8 consecutive lanes over 32 banks (128 bytes;
// measured with single-pattern kernels and SQ_LDS_BANK_CONFLICT). With
// consecutive lanes on consecutive (row, c) the rows of one cycle span two
// 128-byte windows of the tile; rows of the second window store their upper
// half first, so that each cycle fills one window's worth of distinct banks
// (conflict-free for d = 16, 32, 64 at any swizzle of the tile).
template <int D>
__device__ __forceinline__ void st_row_halves(uint16_t* T, int row, int c, const u32x4& lo,
                                              const u32x4& hi) {
  static_assert(D <= 64, "row halves of one 128-byte window");
  constexpr int kRowsPerWindow = 64 / D;
  const bool second = ((row / kRowsPerWindow) & 1) != 0;
  st16(T + tile_off<D>(row, second ? c + D / 16 : c), second ? hi : lo);
  st16(T + tile_off<D>(row, second ? c : c + D / 16), second ? lo : hi);
}

// Lane index computed where it is used: the asm keeps the compiler from
// hoisting it (and values derived from it) out of a loop, where they would
// stay live, or be spilled, across the whole loop.
__device__ __forceinline__ int lane_id_here() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Waits until at most N of this wave's vector-memory operations (which
// include global_load_lds transfers into LDS) are still outstanding; they
// complete in issue order. (s_waitcnt vmcnt(N), other counters untouched.)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Loads two tiles of R rows at once, tile t's row i being global row
// G_t + min(i, lim-1)*rs_t (rows past the valid range repeat the last valid
// one, lim >= 1), into the swizzled LDS tiles T0 and T1. The tiles are
// written in 1 KB pieces, one global_load_lds_dwordx4 per wave and piece
// (lane l fills bytes 16l..16l+15 of the piece); wave w takes pieces
// w, w + 4, w + 8, ... of each tile, so every wave issues the same number of
// loads, LOADS_PER_WAVE. Lane l of piece i covers row i*64/NC + l/NC, chunk
// l % NC: the lane's row is rowbase + ROWSTEP * j for its j-th piece of a
// tile, and as rowbase < ROWSTEP (a power of two) the swizzle of that row is
// swz(rowbase) ^ swz(ROWSTEP * j). A tile of only 2 pieces (R * D = 1024) is
// loaded by waves 0-1 (first tile) and 2-3 (second tile).
template <int D, int R>
struct TilePair {
  static constexpr int NC = D / 8;                 // chunks per row
  static constexpr int PIECES = R * NC / 64;       // per tile
  static constexpr bool SMALL = PIECES == 2;
  static constexpr int PER_TILE = SMALL ? 1 : PIECES / 4;  // pieces per wave and tile
  static constexpr int LOADS_PER_WAVE = SMALL ? 1 : 2 * PER_TILE;
  static constexpr int ROWSTEP = 4 * 64 / NC;      // rows between a wave's pieces
  static_assert(PIECES * 64 == R * NC && (SMALL || PIECES % 4 == 0), "tile shape");

  // Per-lane byte offsets of the copies of a block whose rows all exist (no
  // clamp): computed once per item, so that copies of such blocks take no
  // vector instructions. Row rowbase + ROWSTEP j, chunk xbase ^ swz(ROWSTEP j).
  struct Offsets {
    uint32_t v[PER_TILE];
  };
  __device__ __forceinline__ Offsets offsets(int rs, int w) const {
    const int wp = SMALL ? (w & 1) : w;
    const int lane = __lane_id();
    const int rowbase = wp * (64 / NC) + lane / NC;
    const int xbase = 8 * ((lane % NC) ^ swz<D>(rowbase));
    Offsets o;
#pragma unroll
    for (int j = 0; j < PER_TILE; ++j)
      o.v[j] = 2u * (uint32_t)((rowbase + ROWSTEP * j) * rs + (xbase ^ (8 * swz<D>(ROWSTEP * j))));
    return o;
  }
  // The copies of a block with every row present, from offsets().
  __device__ __forceinline__ void load_full(const uint16_t* __restrict__ G0,
                                            const uint16_t* __restrict__ G1, const Offsets& o,
                                            uint16_t* T0, uint16_t* T1, int w) const {
    const int wp = SMALL ? (w & 1) : w;
    // (the empty asm hands each offset over as a fresh 32-bit value, so that
    // the copy takes the saddr form: uniform base + 32-bit lane offset)
    uint32_t v[PER_TILE];
#pragma unroll
    for (int j = 0; j < PER_TILE; ++j) {
      v[j] = o.v[j];
      asm volatile("" : "+v"(v[j]));
    }
    if (SMALL) {
      const bool second = w >= 2;
      const char* src = reinterpret_cast<const char*>(second ? G1 : G0) + v[0];
      __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)((second ? T1 : T0) + wp * 512), 16,
                                       0, 0);
      return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < PER_TILE; ++j) {
        const char* src = reinterpret_cast<const char*>(t ? G1 : G0) + v[j];
        __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)((t ? T1 : T0) + (wp + 4 * j) * 512),
                                         16, 0, 0);
      }
  }

  // One tile alone (the kernels that stream two tiles of different shapes):
  // wave w takes pieces w, w + 4, ... of it, PER_TILE loads per wave.
  template <int AUX = 0>
  __device__ __forceinline__ void load_one(const uint16_t* __restrict__ G, int rs, int lim,
                                           uint16_t* T, int w) const {
    static_assert(!SMALL, "a tile of at least four pieces");
    const int lane = lane_id_here();
    const int rowbase = w * (64 / NC) + lane / NC;
    const int xbase = 8 * ((lane % NC) ^ swz<D>(rowbase));
#pragma unroll
    for (int j = 0; j < PER_TILE; ++j) {
      const int row = rowbase + ROWSTEP * j;
      const int x = xbase ^ (8 * swz<D>(ROWSTEP * j));
      const uint32_t off = 2u * (uint32_t)(min(row, lim - 1) * rs + x);
      __builtin_amdgcn_global_load_lds((gptr_t)(reinterpret_cast<const char*>(G) + off),
                                       (lptr_t)(T + (w + 4 * j) * 512), 16, 0, AUX);
    }
  }
  __device__ __forceinline__ void load_full_one(const uint16_t* __restrict__ G, const Offsets& o,
                                                uint16_t* T, int w) const {
    static_assert(!SMALL, "a tile of at least four pieces");
#pragma unroll
    for (int j = 0; j < PER_TILE; ++j) {
      uint32_t v = o.v[j];
      asm volatile("" : "+v"(v));  // fresh 32-bit value: the saddr form (see load_full)
      __builtin_amdgcn_global_load_lds((gptr_t)(reinterpret_cast<const char*>(G) + v),
                                       (lptr_t)(T + (w + 4 * j) * 512), 16, 0, 0);
    }
  }

  // Per-lane values of load() are recomputed at each call (a few
  // instructions) rather than kept live across the kernels' main loops.
  __device__ __forceinline__ TilePair(int, int) {}
  // AUX: cache-policy bits of the copies (1 = sc0). A kernel that also
  // copies with load_full passes 1 here: the two call sites then cannot be
  // merged into one copy from a selected 64-bit address.
  template <int AUX = 0>
  __device__ __forceinline__ void load(const uint16_t* __restrict__ G0, int rs0,
                                       const uint16_t* __restrict__ G1, int rs1, int lim,
                                       uint16_t* T0, uint16_t* T1, int w) const {
    const int wp = SMALL ? (w & 1) : w;
    const int lane = lane_id_here();
    const int rowbase = wp * (64 / NC) + lane / NC;
    const int xbase = 8 * ((lane % NC) ^ swz<D>(rowbase));
    // uniform 64-bit base + 32-bit per-lane byte offset (the saddr form)
    if (SMALL) {
      const bool second = w >= 2;
      const uint32_t off =
          2u * (uint32_t)(min(rowbase, lim - 1) * (second ? rs1 : rs0) + xbase);
      const char* src = reinterpret_cast<const char*>(second ? G1 : G0) + off;
      uint16_t* dst = (second ? T1 : T0) + wp * 512;
      __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, AUX);
      return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < PER_TILE; ++j) {
        const int row = rowbase + ROWSTEP * j;
        const int x = xbase ^ (8 * swz<D>(ROWSTEP * j));
        const uint32_t off = 2u * (uint32_t)(min(row, lim - 1) * (t ? rs1 : rs0) + x);
        const char* src = reinterpret_cast<const char*>(t ? G1 : G0) + off;
        uint16_t* dst = (t ? T1 : T0) + (wp + 4 * j) * 512;
        __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, AUX);
      }
    }
  }
};

// LDS slot of 16-byte row entry i (i < 32 within each group of 32): entries
// 16..31 are moved by xor 12, an involution that keeps them in 16..31. A
// lane reads entry perm_row(r); with this placement the lanes of every cycle
// of a ds_read_b128 land on disjoint groups of 4 banks. (Measured with
// single-pattern kernels and SQ_LDS_BANK_CONFLICT on gfx950: the earlier
// xor 8, conflict-free if a cycle served 16 consecutive lanes, costs 4
// extra cycles per read; xor 12 none.)
__device__ __forceinline__ int entry_slot(int i) { return i ^ ((i & 16) ? 12 : 0); }

// Copies the R 16-byte entries src[min(i, lim - 1)], i < R (R = 32 or 64),
// into LDS F at slots entry_slot(i) (4 R dwords): wave w fills dwords
// [w R, w R + R) with one global_load_lds_dword (4 bytes per lane, lanes < R).
__device__ __forceinline__ void load_entries16(const float* __restrict__ src, int R, int lim,
                                               float* F, int w) {
  const int lane = lane_id_here();
  if (lane < R) {
    const int dd = w * R + lane, e = min(entry_slot(dd >> 2), lim - 1);
    const char* p = reinterpret_cast<const char*>(src) + 4u * (uint32_t)(4 * e + (dd & 3));
    __builtin_amdgcn_global_load_lds((gptr_t)p, (lptr_t)(F + w * R), 4, 0, 0);
  }
}

// MFMA operand along d from a tile: lane (r, g) gets logical chunk c of row
// row (8 consecutive d values).
template <int D>
__device__ __forceinline__ u32x4 ld_row(const uint16_t* T, int row, int c) {
  return ld16(T + tile_off<D>(row, c));
}

// MFMA operand rows (ds_read_b128) in one batch: 2*NA reads, a[i] + OA and
// a[i] + OB (immediate byte offsets) for i < NA, into out[0 .. NA) and
// out[NA .. 2 NA), then one wait. Issuing them back to back exposes the LDS
// latency once per batch instead of once per read (left to itself, the
// compiler reuses one 4-register buffer and waits before every MFMA). Inline
// assembly for the same reason as TrRows::read: the compiler would otherwise
// wait for the global_load_lds copies still in flight first; the block waits
// for its own reads (lgkmcnt(0)) before it ends.
template <int NA, int OA, int OB>
__device__ __forceinline__ void lds_rows(const uint32_t (&a)[NA], u32x4 (&out)[2 * NA]) {
  static_assert(OA >= 0 && OB >= 0 && OA < 65536 && OB < 65536, "ds offset field");
  if constexpr (NA == 4) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %1, %9 offset:%12\n\t"
        "ds_read_b128 %5, %9 offset:%13\n\t"
        "ds_read_b128 %2, %10 offset:%12\n\t"
        "ds_read_b128 %6, %10 offset:%13\n\t"
        "ds_read_b128 %3, %11 offset:%12\n\t"
        "ds_read_b128 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]),
          "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OA), "i"(OB)
        : "memory");
  } else if constexpr (NA == 2) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %1, %5 offset:%6\n\t"
        "ds_read_b128 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
        : "v"(a[0]), "v"(a[1]), "i"(OA), "i"(OB)
        : "memory");
  } else {
    static_assert(NA == 1, "1, 2 or 4 rows per operand");
    asm volatile(
        "ds_read_b128 %0, %2 offset:%3\n\t"
        "ds_read_b128 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1])
        : "v"(a[0]), "i"(OA), "i"(OB)
        : "memory");
  }
}

// acc0 += A0 B0 and acc1 += A1 B1 over the NS k-steps (8 d values each) of
// one 32-row MFMA tile, where the A rows of k-step s come from LDS at lane
// byte address a[s] + OFF0 (A0) and a[s] + OFF1 (A1) and the B operands from
// registers: the reads in batches of NA k-steps (lds_rows: 2 NA reads, one
// wait), each accumulator in k-step order.
template <int NS, int NA, int OFF0, int OFF1>
__device__ __forceinline__ void mfma_rows2(const uint32_t (&a)[NS], const u32x4 (&b0)[NS],
                                           const u32x4 (&b1)[NS], f32x16& acc0, f32x16& acc1) {
  static_assert(NS % NA == 0, "whole batches");
#pragma unroll
  for (int h = 0; h < NS / NA; ++h) {
    uint32_t ah[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) ah[i] = a[h * NA + i];
    u32x4 r[2 * NA];
    lds_rows<NA, OFF0, OFF1>(ah, r);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      acc0 = mfma32(r[i], b0[h * NA + i], acc0);
      acc1 = mfma32(r[NA + i], b1[h * NA + i], acc1);
    }
  }
}

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Workgroup barrier without a memory fence: the kernels order their LDS
// traffic themselves (wait_vmem for the global_load_lds copies; every LDS
// read is consumed, hence complete, before the barrier that precedes its
// stage's next copy). The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// MFMA operands whose k index runs along the ROWS of a tile (the transposed
// tile), for the row blocks k0(u) = 32 (u / 2) + 8 (u % 2), u < NU, of the
// 32 columns [32 dt, 32 dt + 32): lane (r = l % 32, g = l / 32) receives
// T[k0 + 16g + e][32 dt + perm_row(r)], e = 0..7, through two
// ds_read_b64_tr_b16 (rows k0 + 16g + 0..3 and + 4..7). That instruction
// works on groups of 16 lanes: lane 4a + b of a group receives element b of
// the 8-byte pieces addressed by lanes a, a+4, a+8, a+12 of the group. Lane s
// of group G addresses row 16g + s/4 (+ k0, + 4) at column
// perm_row(16 (G % 2) + 4 (s % 4)), so lane 4a + b collects four consecutive
// rows of column perm_row(16 (G % 2) + 4a) + b = perm_row(r).
// Row k0 + 16g + s/4 + 4h has the disjoint bits of k0, 16g + s/4 and 4h, and
// swz of the k0 used here is 0, so its swizzle is swz(16g + s/4) ^ swz(4h):
// each lane needs one base address per (h, dt) and the row block is an
// immediate offset. The reads are inline assembly because the compiler,
// unable to tell them apart from the global_load_lds copies still in flight
// into other stages, would otherwise wait for all those copies first; the
// asm block waits for its own reads (lgkmcnt(0)) before it ends.
// ZERO_HI: lanes whose perm_row(r) >= D get zeros (D = 16: tiles narrower
// than 32 columns); their addresses are clamped into the tile.
template <int D>
struct TrRows {
  static constexpr bool ZERO_HI = D < 32;
  static constexpr int ND = D >= 32 ? D / 32 : 1;
  static constexpr int ROWB = 2 * D;  // bytes per tile row
  uint32_t base[2][ND];               // per lane, bytes within the tile
  bool hi_zero;

  __device__ __forceinline__ explicit TrRows(int lane) {
    const int s = lane & 15, G = lane >> 4, g = lane >> 5;
    int col = perm_row(16 * (G & 1) + 4 * (s & 3));
    hi_zero = ZERO_HI && perm_row(lane & 31) >= D;
    if (ZERO_HI && col >= D) col = 0;
    const int rl = 16 * g + (s >> 2);
    const int cx = (col >> 3) ^ swz<D>(rl);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        base[h][dt] = 2 * (rl * D + (col & 7) + 8 * (cx ^ (4 * dt) ^ (h ? swz<D>(4) : 0)));
  }

  // NU operands (NU = 2 or 4) of d tile dt from the tile at LDS byte address
  // tile; one asm block, which returns with the data in registers.
  template <int NU>
  __device__ __forceinline__ void read(uint32_t tile, int dt, u32x4 (&out)[NU]) const {
    const uint32_t b0 = tile + base[0][dt], b1 = tile + base[1][dt];
    u32x2 v[8];
    if constexpr (NU == 4) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
          "ds_read_b64_tr_b16 %1, %9 offset:%11\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
          "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:%14\n\t"
          "ds_read_b64_tr_b16 %5, %9 offset:%15\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:%16\n\t"
          "ds_read_b64_tr_b16 %7, %9 offset:%17\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
            "=&v"(v[6]), "=&v"(v[7])
          : "v"(b0), "v"(b1), "i"(0 * ROWB), "i"(4 * ROWB), "i"(8 * ROWB), "i"(12 * ROWB),
            "i"(32 * ROWB), "i"(36 * ROWB), "i"(40 * ROWB), "i"(44 * ROWB)
          : "memory");
    } else {
      static_assert(NU == 2, "2 or 4 operands");
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
          "ds_read_b64_tr_b16 %1, %5 offset:%7\n\t"
          "ds_read_b64_tr_b16 %2, %4 offset:%8\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:%9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
          : "v"(b0), "v"(b1), "i"(0 * ROWB), "i"(4 * ROWB), "i"(8 * ROWB), "i"(12 * ROWB)
          : "memory");
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      out[u] = u32x4{v[2 * u].x, v[2 * u].y, v[2 * u + 1].x, v[2 * u + 1].y};
      if (ZERO_HI && hi_zero) out[u] = u32x4{0u, 0u, 0u, 0u};
    }
  }
};

}  // namespace esm
