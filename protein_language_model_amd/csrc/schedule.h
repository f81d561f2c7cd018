// Varlen work-item schedule, shared by the device scheduler kernels and the
// host model of them (esm_attn_schedule_host).
//
// Packed batches carry sequences of very different lengths (size-aware bucket
// batching, "BioNeMo Framework" review page, "proposed method"); a work item
// is one block of `block` rows of one (sequence, head) pair, and sequences
// contribute exactly ceil(L / block) items per head, so padding costs nothing.
//
// Order. Sequences are sorted by item count, longest first (so the longest
// items start first and the tail is made of short ones). The (sequence, head)
// "groups" in that order are numbered G = s * H + h and cut into chunks of
// eight consecutive groups. Chunk c owns the slots [base_c, base_c + 8*height_c)
// where height_c is the largest item count among its groups; slot
// base_c + 8*blk + x holds block blk of group 8c + x (idle if that group has
// fewer blocks). base_c is a multiple of 8, so every item of a group lands on
// slots of one residue modulo 8: under round-robin dispatch of workgroups over
// the eight XCDs, all blocks of a (sequence, head) pair run on one XCD and
// share its L2 for their K/V reads.
//
// Launch size. The host cannot read cu_seqlens, so it launches an upper bound
// of slots: 8*NB + H * min(B*NB, floor((T - B')/block) + B'), NB =
// ceil(max_seqlen/block), B' = min(B, T). (height_0 <= NB; for c >= 1,
// height_c is at most the mean of chunk c-1's counts because the order is
// descending, so the sum of heights is at most NB + sum(counts)/8.) Slots past
// the real total are idle.
#pragma once

#include <stdint.h>

namespace esm {

constexpr int kMaxSeqlen = 65536;
constexpr int kMaxBuckets = 4096;   // item counts 0 .. kMaxBuckets-1

#if defined(__HIPCC__)
#define ESM_HD __host__ __device__
#else
#define ESM_HD
#endif

ESM_HD inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Clamped length and start of sequence b (defence against a bad cu_seqlens:
// rows stay inside [0, T)).
ESM_HD inline void seq_bounds(const int32_t* cu, int32_t b, int32_t T, int32_t max_seqlen,
                              int32_t* start, int32_t* len) {
  int32_t s = cu[b], e = cu[b + 1];
  s = s < 0 ? 0 : (s > T ? T : s);
  e = e < s ? s : (e > T ? T : e);
  int32_t L = e - s;
  if (L > max_seqlen) L = max_seqlen;
  *start = s;
  *len = L;
}

ESM_HD inline int64_t schedule_slot_bound(int32_t B, int32_t T, int32_t H, int32_t max_seqlen,
                                          int32_t block) {
  const int64_t nb = ceil_div64(max_seqlen, block);
  const int64_t bp = B < T ? B : T;
  const int64_t by_len = (int64_t)B * nb;
  const int64_t by_tok = (T - bp) / block + bp;
  const int64_t items = by_len < by_tok ? by_len : by_tok;
  return 8 * nb + (int64_t)H * items;
}

ESM_HD inline int64_t schedule_num_chunks(int32_t B, int32_t H) {
  return ceil_div64((int64_t)B * H, 8);
}

// Decode launch slot -> item, given the sorted sequence order and the chunk
// bases (n_chunks + 1 entries, the last one the total slot count).
ESM_HD inline bool schedule_decode(int64_t slot, const int32_t* cu, const int32_t* sorted,
                                   const int32_t* chunk_base, int32_t n_chunks, int32_t B,
                                   int32_t T, int32_t H, int32_t max_seqlen, int32_t block,
                                   int32_t* seq0, int32_t* len, int32_t* head, int32_t* blk) {
  if (n_chunks <= 0 || slot >= chunk_base[n_chunks]) return false;
  int32_t lo = 0, hi = n_chunks - 1;  // largest c with chunk_base[c] <= slot
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (chunk_base[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const int64_t r = slot - chunk_base[lo];
  const int32_t b_blk = (int32_t)(r >> 3);
  const int64_t G = 8 * (int64_t)lo + (r & 7);
  if (G >= (int64_t)B * H) return false;
  const int32_t s = (int32_t)(G / H);
  const int32_t h = (int32_t)(G - (int64_t)s * H);
  int32_t st, L;
  seq_bounds(cu, sorted[s], T, max_seqlen, &st, &L);
  if ((int64_t)b_blk * block >= L) return false;
  *seq0 = st;
  *len = L;
  *head = h;
  *blk = b_blk;
  return true;
}

}  // namespace esm
