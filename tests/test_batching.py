"""Size-aware bucket batching: the oracle (oracle/batching.py) pinned by
hand-worked cases and by the properties the rule fixes, then the library's
host implementation (esm_attn_bucket_batches) equal to it, index for index."""

import bisect
import json
import os

import numpy as np
import pytest

import oracle.batching as OB
from protein_language_model_amd import esm_attn as E

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bucket_batches.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["why"][:40])
def test_oracle_matches_hand_worked_cases(case):
    got = OB.bucket_batches(case["lengths"], case["boundaries"], case["budget"], case["padded"])
    assert got == case["batches"]


def test_bucket_of_is_bisect_right():
    rng = np.random.default_rng(0)
    for _ in range(200):
        bounds = sorted(set(int(x) for x in rng.integers(1, 100, size=rng.integers(0, 6))))
        L = int(rng.integers(0, 120))
        assert OB.bucket_of(L, bounds) == bisect.bisect_right(bounds, L)


def _random_case(rng):
    n = int(rng.integers(0, 60))
    lengths = [int(x) for x in rng.integers(0, 50, size=n)]
    bounds = sorted(set(int(x) for x in rng.integers(1, 50, size=rng.integers(0, 5))))
    budget = int(rng.integers(1, 120))
    padded = bool(rng.integers(0, 2))
    return lengths, bounds, budget, padded


def _check_rule(batches, lengths, bounds, budget, padded):
    """What the rule fixes, checked without re-running it."""
    flat = [i for b in batches for i in b]
    assert sorted(flat) == list(range(len(lengths)))            # every sequence once
    assert all(b for b in batches)                                # no empty batch
    bk = [bisect.bisect_right(bounds, lengths[i]) for i in range(len(lengths))]
    for b in batches:
        assert len({bk[i] for i in b}) == 1                       # one bucket per batch
        if len(b) > 1:                                            # within budget unless alone
            ls = [lengths[i] for i in b]
            cost = len(ls) * max(ls) if padded else sum(ls)
            assert cost <= budget
    # buckets in increasing order; inside a bucket the caller's order
    assert [bk[i] for i in flat] == sorted(bk[i] for i in flat)
    for k in set(bk):
        assert [i for i in flat if bk[i] == k] == [i for i in range(len(lengths)) if bk[i] == k]
    # greedy: a batch closed only because the next sequence of its bucket
    # would have pushed it over the budget
    for b, nxt in zip(batches, batches[1:]):
        if bk[b[0]] == bk[nxt[0]]:
            ls = [lengths[i] for i in b] + [lengths[nxt[0]]]
            cost = len(ls) * max(ls) if padded else sum(ls)
            assert cost > budget


def test_oracle_obeys_the_rule():
    rng = np.random.default_rng(1)
    for _ in range(300):
        lengths, bounds, budget, padded = _random_case(rng)
        _check_rule(OB.bucket_batches(lengths, bounds, budget, padded), lengths, bounds,
                    budget, padded)


def test_padding_and_pair_accounting():
    lengths = [3, 5, 2, 0, 4]
    batches = [[0, 1], [2, 3, 4]]
    # slots: 2*5 + 3*4 = 22, real tokens 14
    assert OB.padding_fraction(batches, lengths) == pytest.approx(1 - 14 / 22)
    assert OB.attention_pairs(batches, lengths, padded=False) == 9 + 25 + 4 + 0 + 16
    assert OB.attention_pairs(batches, lengths, padded=True) == 2 * 25 + 3 * 16
    assert OB.tile_pairs(300, 128, 64) == 3 * 128 * 5 * 64
    assert OB.tile_pairs(128, 128, 64) == 128 * 128
    assert OB.tile_pairs(0, 128, 64) == 0


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["why"][:40])
def test_library_matches_hand_worked_cases(case):
    got = E.esm_attn_bucket_batches(case["lengths"], case["boundaries"], case["budget"],
                                    case["padded"])
    assert [list(map(int, b)) for b in got] == case["batches"]


def test_library_equals_oracle():
    rng = np.random.default_rng(2)
    for _ in range(500):
        lengths, bounds, budget, padded = _random_case(rng)
        got = E.esm_attn_bucket_batches(lengths, bounds, budget, padded)
        assert [list(map(int, b)) for b in got] == OB.bucket_batches(lengths, bounds, budget,
                                                                    padded)


def test_library_at_dataset_scale():
    """A UniRef-like length mix (lognormal, median 300, crop 1024): 20k
    sequences, 64-token buckets, a 16k-token budget, both cost models."""
    rng = np.random.default_rng(3)
    lengths = [int(x) for x in np.clip(np.rint(rng.lognormal(np.log(300), 0.8, 20000)), 30,
                                       1024)]
    bounds = list(range(64, 1024 + 1, 64))
    for padded in (False, True):
        got = [list(map(int, b)) for b in E.esm_attn_bucket_batches(lengths, bounds, 16384,
                                                                    padded)]
        assert got == OB.bucket_batches(lengths, bounds, 16384, padded)
        _check_rule(got, lengths, bounds, 16384, padded)


def test_library_rejects_bad_arguments():
    L = E.lib()
    ln = np.array([3, 4], np.int32)
    order = np.zeros(2, np.int32)
    offs = np.zeros(3, np.int32)
    nb = np.zeros(1, np.int32)
    vp = lambda a: a.ctypes.data
    ok = lambda **kw: L.esm_attn_bucket_batches(
        kw.get("ln", vp(ln)), kw.get("n", 2), kw.get("bd", None), kw.get("nbd", 0),
        kw.get("budget", 10), kw.get("padded", 0), vp(order), vp(offs), kw.get("cap", 2),
        vp(nb))
    assert ok() == E.OK and nb[0] == 1
    assert ok(budget=0) == E.ERR_INVALID_ARGUMENT
    assert ok(padded=2) == E.ERR_INVALID_ARGUMENT
    assert ok(n=-1) == E.ERR_INVALID_ARGUMENT
    assert ok(ln=None) == E.ERR_INVALID_ARGUMENT
    bad = np.array([5, 5], np.int32)
    assert ok(bd=vp(bad), nbd=2) == E.ERR_INVALID_ARGUMENT      # not increasing
    zero = np.array([0], np.int32)
    assert ok(bd=vp(zero), nbd=1) == E.ERR_INVALID_ARGUMENT     # boundary < 1
    neg = np.array([3, -1], np.int32)
    assert ok(ln=vp(neg)) == E.ERR_INVALID_ARGUMENT
    assert ok(budget=3, cap=1) == E.ERR_INVALID_ARGUMENT        # two batches, room for one
