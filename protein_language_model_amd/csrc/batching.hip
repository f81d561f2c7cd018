// Size-aware bucket batching of sequences (host only): the batch former that
// feeds the packed varlen layout. The "BioNeMo Framework" review page lists a
// size-aware batcher and a bucket batch sampler among its components
// ("proposed method") and reports that together they give batches of
// near-uniform size with almost no padding ("main findings"); it gives no
// algorithm. Reading taken here:
//   * buckets: boundaries b_0 < b_1 < ... < b_{K-1} split lengths into K + 1
//     buckets [0, b_0), [b_0, b_1), ..., [b_{K-1}, inf);
//   * size-aware batcher: inside each bucket, sequences are taken in the
//     caller's order and appended to the current batch while the batch's
//     cost stays within the budget; a sequence that would push it over starts
//     the next batch (a sequence over budget on its own is a batch of one).
//     Cost of a batch: its token count (packed layout) or its size times its
//     longest length (padded layout);
//   * batches are emitted bucket by bucket, in the order they were formed.
#include <stdint.h>

#include <vector>

#include "esm_attn.h"

extern "C" esm_attn_status_t esm_attn_bucket_batches(const int32_t* lengths, int32_t n,
                                                     const int32_t* boundaries,
                                                     int32_t n_boundaries, int64_t budget,
                                                     int32_t padded, int32_t* order,
                                                     int32_t* batch_offsets,
                                                     int32_t batch_capacity,
                                                     int32_t* n_batches) {
  if (n < 0 || n_boundaries < 0 || budget < 1 || (padded != 0 && padded != 1) ||
      n_batches == nullptr || batch_offsets == nullptr || batch_capacity < 0 ||
      (n > 0 && (lengths == nullptr || order == nullptr)) ||
      (n_boundaries > 0 && boundaries == nullptr))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  for (int32_t j = 0; j < n_boundaries; ++j)
    if (boundaries[j] < 1 || (j > 0 && boundaries[j] <= boundaries[j - 1]))
      return ESM_ATTN_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n; ++i)
    if (lengths[i] < 0) return ESM_ATTN_ERR_INVALID_ARGUMENT;

  // bucket of each sequence (binary search over the boundaries), then the
  // members of each bucket in input order (counting sort, stable)
  const int32_t nb = n_boundaries + 1;
  std::vector<int32_t> bucket(n), start(nb + 1, 0), members(n);
  for (int32_t i = 0; i < n; ++i) {
    int32_t lo = 0, hi = n_boundaries;  // first boundary > length
    while (lo < hi) {
      const int32_t mid = (lo + hi) / 2;
      if (boundaries[mid] > lengths[i]) hi = mid;
      else lo = mid + 1;
    }
    bucket[i] = lo;
    ++start[lo + 1];
  }
  for (int32_t j = 0; j < nb; ++j) start[j + 1] += start[j];
  {
    std::vector<int32_t> fill(start.begin(), start.end() - 1);
    for (int32_t i = 0; i < n; ++i) members[fill[bucket[i]]++] = i;
  }

  // greedy batches inside each bucket
  int32_t nbat = 0, pos = 0;
  for (int32_t j = 0; j < nb; ++j) {
    int64_t count = 0, sum = 0, longest = 0;
    for (int32_t m = start[j]; m < start[j + 1]; ++m) {
      const int32_t i = members[m];
      const int64_t L = lengths[i];
      const int64_t c1 = count + 1, s1 = sum + L, l1 = L > longest ? L : longest;
      const int64_t cost = padded ? c1 * l1 : s1;
      if (count > 0 && cost > budget) {  // close the current batch
        if (nbat >= batch_capacity) return ESM_ATTN_ERR_INVALID_ARGUMENT;
        batch_offsets[++nbat] = pos;
        count = 1;
        sum = L;
        longest = L;
      } else {
        count = c1;
        sum = s1;
        longest = l1;
      }
      order[pos++] = i;
    }
    if (count > 0) {
      if (nbat >= batch_capacity) return ESM_ATTN_ERR_INVALID_ARGUMENT;
      batch_offsets[++nbat] = pos;
    }
  }
  batch_offsets[0] = 0;
  *n_batches = nbat;
  return ESM_ATTN_OK;
}
