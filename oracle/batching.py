"""Reference for size-aware bucket batching of variable-length sequences, and
the padding and compute accounting of a batch in the packed and padded
layouts.

TEST INFRASTRUCTURE: imported only by tests and the benchmark; never by the
product path.

Source and reading
------------------
The "BioNeMo Framework" review page lists a size-aware batcher and a bucket
batch sampler ("proposed method") and reports that bucketed size-aware
batching gives near-uniform batch sizes with almost no padding ("main
findings"). It prints no algorithm; the plainest reading is taken:

* bucket sampler: increasing boundaries b_0 < ... < b_{K-1} split lengths
  into the buckets [0, b_0), [b_0, b_1), ..., [b_{K-1}, inf);
* size-aware batcher: within a bucket, walk the sequences in the caller's
  order, keeping a current batch; append a sequence if the batch's cost with
  it stays within the budget, otherwise close the batch and open a new one
  holding just that sequence. The cost of a batch is its number of tokens
  (packed layout) or its number of sequences times its longest length
  (padded layout, every sequence padded to the longest);
* the batches come out bucket by bucket, each bucket's in the order formed.

Written as the literal walk, one sequence at a time, with Python lists.
"""


def bucket_of(length, boundaries):
    """Index of the bucket holding `length`: the number of boundaries <= it."""
    k = 0
    for b in boundaries:
        if b <= length:
            k += 1
    return k


def batch_cost(batch_lengths, padded):
    """Tokens of the batch (packed) or size * longest length (padded)."""
    if not batch_lengths:
        return 0
    if padded:
        return len(batch_lengths) * max(batch_lengths)
    return sum(batch_lengths)


def bucket_batches(lengths, boundaries, budget, padded=False):
    """List of batches (lists of indices into `lengths`)."""
    buckets = [[] for _ in range(len(boundaries) + 1)]
    for i, L in enumerate(lengths):
        buckets[bucket_of(L, boundaries)].append(i)
    batches = []
    for members in buckets:
        current = []
        for i in members:
            trial = [lengths[j] for j in current] + [lengths[i]]
            if current and batch_cost(trial, padded) > budget:
                batches.append(current)
                current = [i]
            else:
                current.append(i)
        if current:
            batches.append(current)
    return batches


def padding_fraction(batches, lengths):
    """Share of padded-layout token slots that hold padding:
    1 - sum(L) / sum(batch size * longest length)."""
    real = sum(lengths[i] for b in batches for i in b)
    slots = sum(len(b) * max(lengths[i] for i in b) for b in batches)
    return 1.0 - real / slots if slots else 0.0


def attention_pairs(batches, lengths, padded):
    """(query, key) pairs one attention pass scores: sum of L^2 over the
    sequences when packed; batch size * longest^2 per batch when padded."""
    total = 0
    for b in batches:
        ls = [lengths[i] for i in b]
        if padded:
            total += len(ls) * max(ls) ** 2
        else:
            total += sum(L * L for L in ls)
    return total


def tile_pairs(length, query_rows, key_rows):
    """Pairs a tiled kernel computes for one sequence: whole tiles of
    `query_rows` queries by `key_rows` keys covering the L x L block."""
    nq = -(-length // query_rows)
    nk = -(-length // key_rows)
    return nq * query_rows * nk * key_rows
